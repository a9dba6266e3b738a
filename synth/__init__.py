"""Seeded synthetic inputs for the fused chunked top-K KL loss.

This module is shared by the fp64 oracle tests, the GPU parity tests, the
smoke check and the benchmark.  It holds none of the loss arithmetic: it only
draws hidden states, an output-head weight, a teacher top-K cache and a token
mask with the shapes and value distributions of the workloads below, and rounds
h and W to bf16 (round-to-nearest-even) so that both sides see the same bits.

The teacher cache mimics an offline top-K cache (page "Making Knowledge
Distillation Cheap Enough to Run at Scale", section "Two systems changes",
paragraph on offline distillation): per position, the K largest logits of a
teacher and their vocabulary indices.  No teacher model exists here, so the
teacher logits are the student's own logits plus unit Gaussian noise; the top-K
per row is kept sorted by value (descending), ties broken by the lower index.

Workloads (head shapes of the page's gpt-oss and Qwen examples):
  tiny    T=128    H=256  V=4096   K=32  tau=1  (fp32 values; bf16 for GPU parity)
  gptoss  T=4096   H=2880 V=201088 K=64  tau=1
  long    T=32768  H=2880 V=201088 K=64  tau=2  packed 8-document mask
  qwen    T=16384  H=4096 V=151936 K=128 tau=1  10% random padding
  sweep   T in {4096,16384,65536,131072,262144}, H=2880 V=201088 K=64
"""
from __future__ import annotations

import dataclasses
import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "SWEEP_T", "round_bf16_np", "bf16_bits_np",
    "make_mask_np", "make_inputs_np", "make_inputs_torch",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    V: int
    K: int
    tau: float
    mask: str = "ones"       # "ones" | "packed8" | "pad10"
    chunk_v: int = 0         # 0 = library default


WORKLOADS = {
    "tiny": Workload("tiny", 128, 256, 4096, 32, 1.0, "ones", 1024),
    "gptoss": Workload("gptoss", 4096, 2880, 201088, 64, 1.0, "ones"),
    "long": Workload("long", 32768, 2880, 201088, 64, 2.0, "packed8"),
    "qwen": Workload("qwen", 16384, 4096, 151936, 128, 1.0, "pad10"),
}
SWEEP_T = (4096, 16384, 65536, 131072, 262144)

# stream ids for Generator(PCG64(1000*seed + stream))
_S_H, _S_W, _S_NOISE, _S_MASK = 0, 1, 2, 3


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(1000 * int(seed) + stream))


def bf16_bits_np(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round-to-nearest-even.
    Inputs here are finite, so no NaN special case is needed."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def round_bf16_np(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bf16 (RNE), returned as float32."""
    b = bf16_bits_np(x).astype(np.uint32) << 16
    return b.view(np.float32)


def make_mask_np(T: int, kind: str, seed: int) -> np.ndarray:
    """uint8 [T] mask; 1 = position counts toward the loss.

    ones    : all positions kept.
    packed8 : 8 packed documents of random lengths summing to T; the first
              token of each document is masked (7 distinct cut points drawn
              uniformly from [1, T-1], plus position 0).
    pad10   : round(0.1*T) positions, uniform without replacement, masked.
    """
    m = np.ones(T, dtype=np.uint8)
    if T == 0 or kind == "ones":
        return m
    r = _rng(seed, _S_MASK)
    if kind == "packed8":
        ndoc = 8
        cuts = np.sort(r.choice(np.arange(1, T), size=min(ndoc - 1, T - 1), replace=False))
        m[0] = 0
        m[cuts] = 0
        return m
    if kind == "pad10":
        n = int(round(0.1 * T))
        m[r.choice(T, size=n, replace=False)] = 0
        return m
    raise ValueError(f"unknown mask kind {kind!r}")


def _topk_rows_np(S: np.ndarray, K: int):
    """Per row: K largest values, sorted descending, ties -> lower index first."""
    T, V = S.shape
    # lexsort on (index asc) then (value desc): primary key is the last one
    cols = np.arange(V)[None, :].repeat(T, 0)
    order = np.lexsort((cols, -S), axis=1)[:, :K]
    vals = np.take_along_axis(S, order, axis=1)
    return order.astype(np.int32), vals.astype(np.float32)


def make_inputs_np(T: int, H: int, V: int, K: int, seed: int = 0, *,
                   bf16: bool = True, mask: str = "ones",
                   teacher_noise: float = 1.0, logit_scale: float = 2.0) -> dict:
    """Host (numpy) inputs, for shapes the CPU can draw in seconds.

    h ~ N(0,1) [T,H]; W ~ logit_scale*N(0,1)/sqrt(H) [V,H] (student logits
    std ~ logit_scale: 2 for the workloads, ~10-15 for sharp softmaxes);
    teacher logits = h.W^T (fp32) + teacher_noise*N(0,1); top-K per row.
    With bf16=True h and W are rounded to bf16 first and the teacher is built
    from the rounded values; 'h_bits'/'W_bits' carry the uint16 patterns.
    """
    h = _rng(seed, _S_H).standard_normal((T, H), dtype=np.float32)
    W = (_rng(seed, _S_W).standard_normal((V, H), dtype=np.float32)
         * np.float32(logit_scale / np.sqrt(H)))
    if bf16:
        h = round_bf16_np(h)
        W = round_bf16_np(W)
    S = h @ W.T
    S = S + np.float32(teacher_noise) * _rng(seed, _S_NOISE).standard_normal(S.shape, dtype=np.float32)
    idx, logit = _topk_rows_np(S, K)
    out = dict(h=h, W=W, teacher_idx=idx, teacher_logit=logit,
               mask=make_mask_np(T, mask, seed))
    if bf16:
        out["h_bits"] = bf16_bits_np(h)
        out["W_bits"] = bf16_bits_np(W)
    return out


def make_inputs_torch(T: int, H: int, V: int, K: int, seed: int = 0, *,
                      device="cuda", mask: str = "ones", teacher_noise: float = 1.0,
                      row_chunk: int = 2048, logit_scale: float = 2.0) -> dict:
    """Device inputs for the large workloads (torch is used as a random-number
    and matmul engine here; none of this is the loss).  h, W bf16; teacher
    top-K built in row chunks from bf16 h.W^T (fp32 accumulate) + noise, each
    chunk seeded as seed*1_000_003 + chunk.  Same distributions as
    make_inputs_np (different random streams)."""
    import torch
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(1000 * seed + _S_H)
    h = torch.randn((T, H), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    g.manual_seed(1000 * seed + _S_W)
    W = (torch.randn((V, H), generator=g, device=dev, dtype=torch.float32)
         * (logit_scale / np.sqrt(H))).to(torch.bfloat16)
    idx = torch.empty((T, K), dtype=torch.int32, device=dev)
    val = torch.empty((T, K), dtype=torch.float32, device=dev)
    for c, t0 in enumerate(range(0, T, row_chunk)):
        t1 = min(T, t0 + row_chunk)
        S = torch.nn.functional.linear(h[t0:t1], W).float()
        g.manual_seed(seed * 1_000_003 + c)
        S += teacher_noise * torch.randn(S.shape, generator=g, device=dev, dtype=torch.float32)
        # descending values; torch.topk on distinct continuous values has no ties
        v, i = torch.topk(S, K, dim=1, largest=True, sorted=True)
        idx[t0:t1] = i.to(torch.int32)
        val[t0:t1] = v
        del S
    m = torch.from_numpy(make_mask_np(T, mask, seed)).to(dev)
    return dict(h=h, W=W, teacher_idx=idx, teacher_logit=val, mask=m)
