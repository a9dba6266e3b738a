"""Benchmark of the fused chunked top-K KL loss (forward + backward) on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gptoss]

One step = one kd_topk_kl_fwd_bwd call (teacher prep, gather, pass 1
log-sum-exp, loss, pass 2 recompute + logit gradient + dH/dW contractions)
over one synthetic batch already resident in HBM.  Prints one JSON line;
its "seq_chunk" object times the same call under the sequence-chunk
schedule (stored block logits instead of the pass-2 recompute), and
"logits_variant" the forward-chunked KL on the batch's materialised logits.

Other modes (not the benchmark line):
  --copy-probe      a plain device copy of known size, to calibrate rocprofv3
                    FETCH_SIZE / WRITE_SIZE against the algorithmic bytes
  --sweep           tokens/s and peak memory over T in {4096 ... 262144}
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "tokens/s fwd+bwd fused chunked KL (H=2880,V=201088,K=64); MFMA util; peak mem"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "bwd_traffic_gptoss.json")
# the sources k_bwd is built and launched from (the traffic summary is its)
KERNEL_SOURCES = [os.path.join(ROOT, "chunked_kl_loss_02_amd", "csrc", f)
                  for f in ("kd_common.hpp", "kd_gemm.hpp", "kd_kernels.hpp", "kd_host.hip")]


def naive_logit_bytes(T: int, V: int, itemsize: int = 2) -> int:
    """Bytes of one dense [T, V] logit (or teacher-probability) tensor."""
    return int(T) * int(V) * int(itemsize)


def flops_per_token(H: int, V: int) -> float:
    """Algorithmic MFMA work per token: pass-1 GEMM, pass-2 recompute, dH and
    dW contractions, 2*H*V each."""
    return 8.0 * H * V


def kernel_source_hash() -> str:
    """Hash of the kernel sources with comments and whitespace removed, so
    that the committed traffic counters stay attached to the code they were
    measured on (and only to it)."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update("".join(text.split()).encode())
    return h.hexdigest()[:16]


def cpu_baseline(x, tau, rows: int, seed: int = 0):
    """Times the fp64 oracle (as it stands) on `rows` sampled tokens of the
    workload: full vocabulary forward, loss, dH rows and dW."""
    import numpy as np
    import torch
    from oracle import kl_dense
    T = x["h"].shape[0]
    sel = np.sort(np.random.default_rng(seed).choice(T, size=min(rows, T), replace=False))
    st = torch.from_numpy(sel).to(x["h"].device)
    h = x["h"].index_select(0, st).float().cpu().numpy()
    W = x["W"].float().cpu().numpy()
    idx = x["teacher_idx"].index_select(0, st).cpu().numpy()
    lg = x["teacher_logit"].index_select(0, st).cpu().numpy()
    m = x["mask"].index_select(0, st).cpu().numpy()
    cores = len(os.sched_getaffinity(0))
    from threadpoolctl import threadpool_limits, threadpool_info
    with threadpool_limits(limits=cores):
        used = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        t0 = time.perf_counter()
        kl_dense(h, W, idx, lg, m, tau)
        dt = time.perf_counter() - t0
    return {"value": len(sel) / dt, "unit": "tokens/s", "cores": int(used), "kind": "oracle",
            "sample": f"{len(sel)} of {T} tokens (seeded), full V={x['W'].shape[0]}, loss + dH rows + dW in fp64",
            "seconds": dt}


def load_traffic(launch_flops):
    """HBM bytes per bwd launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel sources; else None."""
    try:
        with open(PROFILE_TRAFFIC) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def run_seq_chunk(args, wl, x):
    """The sequence-chunk schedule on the same inputs: pass 1 keeps a token
    block's logits (fp32, in the workspace) and the gradient is formed from
    them, 6 T H V flops instead of 8.  Reported beside the main line."""
    import torch
    import chunked_kl_loss_02_amd as kd
    dev = x["h"].device
    T, H, V, K, tau = wl.T, wl.H, wl.V, wl.K, wl.tau
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    ws_bytes = kd.workspace_size(T, H, V, K, tau, seq_chunk=True)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    outs = (torch.empty((), dtype=torch.float32, device=dev),
            torch.empty((T, H), dtype=torch.float32, device=dev),
            torch.empty((V, H), dtype=torch.float32, device=dev))

    def step():
        return kd.fwd_bwd(x["h"], x["W"], x["teacher_idx"], x["teacher_logit"], x["mask"], tau,
                          workspace=ws, out=outs, seq_chunk=True)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    dt, pk = timed_steps(step, args.steps, ["bwd"])
    peak = torch.cuda.max_memory_allocated(dev)
    bwd_ms, bwd_n = pk["bwd"]
    _, per_kernel = timed_steps(step, args.steps)
    res = {
        "value": T * args.steps / dt, "unit": "tokens/s", "ms_per_step": dt * 1e3 / args.steps,
        "flops_per_token": 6.0 * H * V,
        "tflops": 6.0 * H * V * T * args.steps / dt / 1e12,
        "bwd_achieved_tflops": 4.0 * T * H * V * args.steps / (bwd_ms * 1e-3) / 1e12 if bwd_ms > 0 else 0.0,
        "per_kernel_ms_per_step": {k: v[0] / args.steps for k, v in per_kernel.items() if v[1]},
        "peak_mem_bytes": int(peak), "workspace_bytes": int(ws_bytes),
        "loss": outs[0].item(),
    }
    del ws, outs
    torch.cuda.empty_cache()
    return res


def timed_steps(step, steps, classes=None):
    """Runs `steps` calls of step() between two device synchronisations;
    returns (seconds, {class: (ms, launches)}) with HIP events recorded only
    around the launches of `classes` (None: every class)."""
    import torch
    import chunked_kl_loss_02_amd as kd
    kd.timing_enable(True, classes)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    kd.timing_enable(False)
    return dt, kd.timing_collect()


def run_logits_variant(args, wl, x):
    """Forward-chunked KL on the materialised bf16 logits of the same batch
    (Z = h W^T): loss + dZ.  HBM-bound: the algorithmic traffic is one read
    and one write of Z, 4 bytes per logit (the kernel's second read of a row
    mostly hits the last-level cache)."""
    import torch
    import chunked_kl_loss_02_amd as kd
    T, V = wl.T, wl.V
    Z = torch.nn.functional.linear(x["h"], x["W"])
    dZ = torch.empty_like(Z)
    loss = torch.empty((), dtype=torch.float32, device=Z.device)
    ws = torch.empty(kd.logits_workspace_size(T, V, wl.K, wl.tau), dtype=torch.uint8, device=Z.device)

    def step():
        kd.kl_logits(Z, x["teacher_idx"], x["teacher_logit"], x["mask"], wl.tau, workspace=ws, out=(loss, dZ))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    dt, pk = timed_steps(step, args.steps)
    row_ms, row_n = pk["logits"]
    bytes_step = 4.0 * T * V
    res = {"value": T * args.steps / dt, "unit": "tokens/s", "ms_per_step": dt * 1e3 / args.steps,
           "roofline": {"bound": "hbm", "kernel": "k_lrow (row log-sum-exp + dZ)",
                        "achieved": bytes_step * row_n / (row_ms * 1e-3) / 1e9 if row_ms > 0 else 0.0,
                        "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": bytes_step * row_n / (row_ms * 1e-3) / 1e9 / PEAK_HBM_GBS if row_ms > 0 else 0.0,
                        "bytes_per_launch": bytes_step, "avg_launch_ms": row_ms / max(row_n, 1)},
           "per_kernel_ms_per_step": {k: v[0] / args.steps for k, v in pk.items() if v[1]},
           "loss": loss.item()}
    # the teacher-cache producer on the same [T, V] bf16 grid: top-K per row
    idx = torch.empty((T, wl.K), dtype=torch.int32, device=Z.device)
    val = torch.empty((T, wl.K), dtype=torch.float32, device=Z.device)
    for _ in range(args.warmup):
        kd.topk_select(Z, wl.K, out=(idx, val))
    torch.cuda.synchronize()
    dt, pk = timed_steps(lambda: kd.topk_select(Z, wl.K, out=(idx, val)), args.steps)
    tk_ms, tk_n = pk["topk"]
    tk_bytes = 2.0 * T * V + 8.0 * T * wl.K
    res["topk_variant"] = {
        "value": T * args.steps / dt, "unit": "rows/s", "ms_per_step": dt * 1e3 / args.steps, "K": wl.K,
        "roofline": {"bound": "hbm", "kernel": "k_topk (per-row top-K of bf16 logits)",
                     "achieved": tk_bytes * tk_n / (tk_ms * 1e-3) / 1e9 if tk_ms > 0 else 0.0, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": tk_bytes * tk_n / (tk_ms * 1e-3) / 1e9 / PEAK_HBM_GBS if tk_ms > 0 else 0.0,
                     "bytes_per_launch": tk_bytes, "avg_launch_ms": tk_ms / max(tk_n, 1)}}
    del Z, dZ, ws, idx, val
    torch.cuda.empty_cache()
    return res


def run_one(args, wl):
    import numpy as np
    import torch
    import chunked_kl_loss_02_amd as kd
    import synth
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    T, H, V, K, tau = wl.T, wl.H, wl.V, wl.K, wl.tau
    x = synth.make_inputs_torch(T, H, V, K, seed=args.seed, device=dev, mask=wl.mask)
    torch.cuda.synchronize()
    ws_bytes = kd.workspace_size(T, H, V, K, tau)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    outs = (torch.empty((), dtype=torch.float32, device=dev),
            torch.empty((T, H), dtype=torch.float32, device=dev),
            torch.empty((V, H), dtype=torch.float32, device=dev))

    def step():
        return kd.fwd_bwd(x["h"], x["W"], x["teacher_idx"], x["teacher_logit"], x["mask"], tau,
                          workspace=ws, out=outs)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    base_alloc = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    # the timed region: events only around the roofline kernel's launches
    dt, pk = timed_steps(step, args.steps, ["bwd"])
    peak = torch.cuda.max_memory_allocated(dev)
    loss = outs[0].item()
    ms_step = dt * 1e3 / args.steps
    bwd_ms, bwd_n = pk["bwd"]
    # per-kernel breakdown: the same steps again, events around every launch
    dt_all, per_kernel = timed_steps(step, args.steps)
    bwd_flops_total = 4.0 * T * H * V * args.steps       # dH + dW contractions
    achieved = bwd_flops_total / (bwd_ms * 1e-3) / 1e12 if bwd_ms > 0 else 0.0
    traffic = load_traffic(bwd_flops_total / max(bwd_n, 1))
    res = {
        "metric": METRIC,
        "value": T * args.steps / dt,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded h~N(0,1), W~2N(0,1)/sqrt(H), teacher top-K of noisy student logits)",
        "config": {"workload": wl.name, "T": T, "H": H, "V": V, "K": K, "tau": tau, "mask": wl.mask,
                   "seq_len": T, "global_batch": 1, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "kernel": "k_bwd (dH = G W_c and dW_c = G^T h, bf16 MFMA)",
                     "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
                     "avg_launch_ms": bwd_ms / max(bwd_n, 1), "launches": bwd_n},
        "tflops_total": flops_per_token(H, V) * T * args.steps / dt / 1e12,
        "mfma_util_total": flops_per_token(H, V) * T * args.steps / dt / 1e12 / PEAK_BF16_TFLOPS,
        "per_kernel_ms_per_step": {k: v[0] / args.steps for k, v in per_kernel.items() if v[1]},
        "ms_per_step_all_events": dt_all * 1e3 / args.steps,
        "peak_mem_bytes": int(peak),
        "peak_mem_inputs_outputs_workspace_bytes": int(base_alloc),
        "workspace_bytes": int(ws_bytes),
        "naive_logits_bytes": naive_logit_bytes(T, V),
        "loss": loss,
    }
    return res, x


def copy_probe(nbytes=1 << 30, reps=5):
    """Plain device-to-device copy of nbytes, for counter calibration."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "reps": reps}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--workload", default="gptoss", choices=["gptoss", "long", "qwen", "tiny"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-seq-chunk", action="store_true", help="skip the sequence-chunk schedule line")
    ap.add_argument("--no-variants", action="store_true", help="skip the logits / top-K variant lines")
    ap.add_argument("--cpu-rows", type=int, default=2048)
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--sweep", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the loss would shard along tokens). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe()
        return
    import synth
    if args.sweep:
        for T in synth.SWEEP_T:
            wl = synth.Workload(f"sweep-T{T}", T, 2880, 201088, 64, 1.0)
            res, x = run_one(args, wl)
            del x
            res.pop("roofline", None)
            print(json.dumps(res), flush=True)
        return
    wl = synth.WORKLOADS[args.workload]
    res, x = run_one(args, wl)
    res["config"]["schedule"] = "recompute (pass 2 recomputes each vocabulary chunk)"
    if not args.no_seq_chunk:
        res["seq_chunk"] = run_seq_chunk(args, wl, x)
    if not args.no_variants:
        res["logits_variant"] = run_logits_variant(args, wl, x)
        res["topk_variant"] = res["logits_variant"].pop("topk_variant")
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(x, wl.tau, args.cpu_rows)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
