"""Benchmark of the fused chunked top-K KL loss (forward + backward) on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gptoss]

One step = one kd_topk_kl_fwd_bwd call (teacher prep, gather, pass 1
log-sum-exp, loss, pass 2 recompute + logit gradient + dH/dW contractions)
over one synthetic batch already resident in HBM.  Prints one JSON line;
its "seq_chunk" object times the same call under the sequence-chunk
schedule (stored block logits instead of the pass-2 recompute), and
"logits_variant" the forward-chunked KL on the batch's materialised logits.

Other modes (not the benchmark line):
  --copy-probe      a plain device copy of known size, to check rocprofv3
                    byte counts against the algorithmic bytes
  --summarize-counters DIR WORKLOAD OUT
                    per-kernel L2-to-fabric bytes from rocprofv3 --pmc passes
  --sweep           tokens/s and peak memory over T in {4096 ... 262144}
                    (the default run already carries them in "scaling")

The default run also adds "scaling": the long-context head (T 32768, tau 2,
packed mask), the Qwen-like head and the output-head sweep T in {16384,
65536, 131072, 262144}, each with tokens/s, TFLOP/s over 8 T H V, peak device
memory and the naive 2 T V logit bytes; and, in "cpu_baseline", the tiny
config timed in full through the oracle at one thread and at every core.
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
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "bwd_pass2_traffic_gptoss.json")
ROOFLINE_KERNEL = "k_bwd_pass2"
# the sources the roofline kernel is built and launched from (the traffic
# summary is attached to them)
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


def load_traffic():
    """(bytes per launch, what they count) of the roofline kernel from the
    committed rocprofv3 counter summary, if it was taken on the current
    kernel sources; else (None, reason)."""
    try:
        with open(PROFILE_TRAFFIC) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None, "no counter summary"
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None, "counter summary taken on other kernel sources"
    k = d["kernels"].get(ROOFLINE_KERNEL)
    if not k:
        return None, "roofline kernel missing from the counter summary"
    return k["read_bytes"] + k["write_bytes"], d["counts"]


def merged_flops(T, H, V, K, tau):
    """MFMA flops of the k_bwd_pass2 launches of one call and their number:
    launch i holds unit i's dH and dW contractions (4 H rows_i vrows_i) and
    unit i+1's pass-2 recompute (2 H rows_{i+1} vrows_{i+1}); units are
    (token block, vocabulary chunk) pairs in the library's order, the last
    unit's contractions launch alone (k_bwd)."""
    import chunked_kl_loss_02_amd as kd
    bt, cv, nbuf = kd.tiling(T, H, V, K, tau)
    units = [(min(bt, T - t0), min(cv, V - v0)) for t0 in range(0, T, bt) for v0 in range(0, V, cv)]
    if nbuf < 2:
        return 0.0, 0
    f = sum(4.0 * H * r * v + 2.0 * H * units[i + 1][0] * units[i + 1][1] for i, (r, v) in enumerate(units[:-1]))
    return f, len(units) - 1


def kernel_flops(T, H, V, K, tau):
    """MFMA flops per call of each GEMM kernel class of the recompute
    schedule, from the library's (token block, vocabulary chunk) units:
    pass 1 computes every logit once (2 H per logit); with two gradient
    buffers the first unit's pass 2 runs alone (pass2), the merged launches
    hold the rest (bwd_pass2, see merged_flops) and the last unit's
    contractions run alone (bwd); with one buffer every unit's pass 2 and
    contractions run as pass2 and bwd."""
    import chunked_kl_loss_02_amd as kd
    bt, cv, nbuf = kd.tiling(T, H, V, K, tau)
    units = [(min(bt, T - t0), min(cv, V - v0)) for t0 in range(0, T, bt) for v0 in range(0, V, cv)]
    out = {"pass1": 2.0 * T * H * V}
    if nbuf < 2:
        out["pass2"] = sum(2.0 * H * r * v for r, v in units)
        out["bwd"] = sum(4.0 * H * r * v for r, v in units)
    else:
        out["pass2"] = 2.0 * H * units[0][0] * units[0][1]
        out["bwd"] = 4.0 * H * units[-1][0] * units[-1][1]
        out["bwd_pass2"] = merged_flops(T, H, V, K, tau)[0]
    return out


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
    dt, pk = timed_steps(step, args.steps, ["bwd", "bwd_pass2"])
    peak = torch.cuda.max_memory_allocated(dev)
    # every contraction of this schedule runs in k_bwd_sgrad (class bwd_pass2,
    # which also forms the next chunk's gradient tiles) or k_bwd (last chunk)
    grad_ms = pk["bwd"][0] + pk["bwd_pass2"][0]
    _, per_kernel = timed_steps(step, args.steps)
    res = {
        "value": T * args.steps / dt, "unit": "tokens/s", "ms_per_step": dt * 1e3 / args.steps,
        "flops_per_token": 6.0 * H * V,
        "tflops": 6.0 * H * V * T * args.steps / dt / 1e12,
        "contraction_launches_tflops": 4.0 * T * H * V * args.steps / (grad_ms * 1e-3) / 1e12 if grad_ms > 0 else 0.0,
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
    dt, pk = timed_steps(step, args.steps, ["bwd_pass2"])
    peak = torch.cuda.max_memory_allocated(dev)
    loss = outs[0].item()
    ms_step = dt * 1e3 / args.steps
    mg_ms, mg_n = pk["bwd_pass2"]
    # per-kernel breakdown: the same steps again, events around every launch
    dt_all, per_kernel = timed_steps(step, args.steps)
    mg_flops, mg_launches = merged_flops(T, H, V, K, tau)
    achieved = mg_flops * args.steps / (mg_ms * 1e-3) / 1e12 if mg_ms > 0 else 0.0
    traffic, traffic_kind = load_traffic()
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
        "roofline": {"bound": "mfma",
                     "kernel": "k_bwd_pass2 (dH = G W_c and dW_c = G^T h of one (block, chunk) unit and the next "
                               "unit's pass-2 recompute, bf16 MFMA)",
                     "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic, "traffic_kind": traffic_kind,
                     "flops_per_launch": mg_flops / max(mg_launches, 1),
                     "avg_launch_ms": mg_ms / max(mg_n, 1), "launches": mg_n},
        "tflops_total": flops_per_token(H, V) * T * args.steps / dt / 1e12,
        "mfma_util_total": flops_per_token(H, V) * T * args.steps / dt / 1e12 / PEAK_BF16_TFLOPS,
        "per_kernel_ms_per_step": {k: v[0] / args.steps for k, v in per_kernel.items() if v[1]},
        # MFMA rate of each GEMM kernel class over its event-timed share of a step
        "per_kernel_tflops": {k: f * args.steps / (per_kernel[k][0] * 1e-3) / 1e12
                              for k, f in kernel_flops(T, H, V, K, tau).items()
                              if k in per_kernel and per_kernel[k][1] and per_kernel[k][0] > 0},
        "ms_per_step_all_events": dt_all * 1e3 / args.steps,
        "peak_mem_bytes": int(peak),
        "peak_mem_inputs_outputs_workspace_bytes": int(base_alloc),
        "workspace_bytes": int(ws_bytes),
        "naive_logits_bytes": naive_logit_bytes(T, V),
        "loss": loss,
    }
    return res, x


def run_scaling_point(args, wl, steps, warmup):
    """One fused call per step at a larger workload (same kernels and default
    tiling as the main line): tokens/s, TFLOP/s over 8 T H V, peak device
    memory of the call (inputs, outputs, workspace) against the 2 T V bytes
    of one bf16 logit tensor, and the gradient contractions' rate."""
    import torch
    import chunked_kl_loss_02_amd as kd
    import synth
    dev = torch.device("cuda:0")
    T, H, V, K, tau = wl.T, wl.H, wl.V, wl.K, wl.tau
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    x = synth.make_inputs_torch(T, H, V, K, seed=args.seed, device=dev, mask=wl.mask)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    base = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    ws_bytes = kd.workspace_size(T, H, V, K, tau)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    outs = (torch.empty((), dtype=torch.float32, device=dev),
            torch.empty((T, H), dtype=torch.float32, device=dev),
            torch.empty((V, H), dtype=torch.float32, device=dev))

    def step():
        return kd.fwd_bwd(x["h"], x["W"], x["teacher_idx"], x["teacher_logit"], x["mask"], tau,
                          workspace=ws, out=outs)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    dt, pk = timed_steps(step, steps, ["bwd_pass2"])
    peak = torch.cuda.max_memory_allocated(dev)
    inputs = sum(t.numel() * t.element_size() for t in x.values())
    mg_ms, _ = pk["bwd_pass2"]
    mg_flops, _ = merged_flops(T, H, V, K, tau)
    flops = flops_per_token(H, V) * T
    res = {"workload": wl.name, "T": T, "H": H, "V": V, "K": K, "tau": tau, "mask": wl.mask,
           "kept_tokens": int(x["mask"].sum().item()), "steps": steps, "warmup": warmup,
           "value": T * steps / dt, "unit": "tokens/s", "ms_per_step": dt * 1e3 / steps,
           "tflops": flops * steps / dt / 1e12, "mfma_frac": flops * steps / dt / 1e12 / PEAK_BF16_TFLOPS,
           "bwd_pass2_tflops": mg_flops * steps / (mg_ms * 1e-3) / 1e12 if mg_ms > 0 else 0.0,
           "peak_mem_bytes": int(peak - base + inputs), "workspace_bytes": int(ws_bytes),
           "naive_logits_bytes": naive_logit_bytes(T, V), "loss": outs[0].item()}
    del x, ws, outs
    torch.cuda.empty_cache()
    return res


def scaling_lines(args):
    """The output-head scaling sweep (single sequences, H2880 V201088 K64)
    and the long-context and Qwen-like heads, each timed by the same clock
    as the main line; fewer steps at the largest T."""
    import synth
    out = []
    pts = [synth.WORKLOADS["long"], synth.WORKLOADS["qwen"]]
    pts += [synth.Workload(f"sweep-T{T}", T, 2880, 201088, 64, 1.0) for T in synth.SWEEP_T if T != 4096]
    for wl in pts:
        steps = 5 if wl.T <= 32768 else 3 if wl.T <= 65536 else 2
        r = run_scaling_point(args, wl, steps, 1)
        print(f"[scaling] {wl.name}: {r['value']:.4g} tokens/s, {r['ms_per_step']:.1f} ms/step, "
              f"peak {r['peak_mem_bytes'] / 1e9:.2f} GB", file=sys.stderr, flush=True)
        out.append(r)
    return out


def cpu_tiny_full(seconds=3.0):
    """The tiny config (T128 H256 V4096 K32, tau 1), whole problem, through
    the fp64 oracle: loss, dH and dW, at one BLAS thread and at every core
    of this host; repeated for about `seconds` each."""
    import synth
    from oracle import kl_dense
    from threadpoolctl import threadpool_limits, threadpool_info
    wl = synth.WORKLOADS["tiny"]
    x = synth.make_inputs_np(wl.T, wl.H, wl.V, wl.K, seed=1, bf16=False)
    cores = len(os.sched_getaffinity(0))
    res = {"workload": "tiny T128 H256 V4096 K32 tau1 (fp32 inputs, whole problem, loss + dH + dW)",
           "unit": "tokens/s", "kind": "oracle"}
    for key, lim in (("one_thread", 1), ("all_cores", cores)):
        with threadpool_limits(limits=lim):
            used = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
            n, t0 = 0, time.perf_counter()
            while True:
                kl_dense(x["h"], x["W"], x["teacher_idx"], x["teacher_logit"], x["mask"], wl.tau)
                n += 1
                dt = time.perf_counter() - t0
                if dt >= seconds:
                    break
        res[key] = {"value": wl.T * n / dt, "cores": int(used), "calls": n, "seconds": dt}
    return res


def summarize_counters(pmc_dir, workload, out_json):
    """Per-kernel bytes per dispatch from four rocprofv3 --pmc passes over the
    same program (directories pmc_dir/{A,B,C,D}, files <workload>_counter_collection.csv):
      A  TCC_EA0_RDREQ_32B_sum TCC_EA0_RDREQ_64B_sum TCC_EA0_RDREQ_128B_sum TCC_EA0_RDREQ_sum
      B  TCC_EA0_WRREQ_sum TCC_EA0_WRREQ_64B_sum TCC_EA0_RDREQ_DRAM_32B_sum TCC_EA0_WRREQ_DRAM_sum
      C  FETCH_SIZE        D  WRITE_SIZE
    read = 32 n32 + 64 n64 + 128 n128 (the L2's read requests to the fabric by
    size), write = 32 (nW - nW64) + 64 nW64; FETCH_SIZE and WRITE_SIZE are
    kept beside them as a cross-check.  These count bytes between the L2
    and the memory fabric: last-level (Infinity) cache hits are included,
    so they bound HBM traffic from above."""
    import csv
    import collections
    def load(pas):
        path = os.path.join(pmc_dir, pas, f"{workload}_counter_collection.csv")
        acc = collections.defaultdict(lambda: collections.defaultdict(float))
        disp = collections.defaultdict(set)
        for r in csv.DictReader(open(path)):
            m = re.search(r"\bkd::(k_\w+)", r["Kernel_Name"])
            name = m.group(1) if m else "other:" + r["Kernel_Name"][:40]
            acc[name][r["Counter_Name"]] += float(r["Counter_Value"])
            disp[name].add(r["Dispatch_Id"])
        return {k: ({c: v / len(disp[k]) for c, v in acc[k].items()}, len(disp[k])) for k in acc}
    A, B, C, D = (load(p) for p in "ABCD")
    kernels = {}
    for k, (a, n) in A.items():
        if k.startswith("other:"):
            continue
        b, c, d = B[k][0], C.get(k, ({}, 0))[0], D.get(k, ({}, 0))[0]
        rd = 32 * a["TCC_EA0_RDREQ_32B_sum"] + 64 * a["TCC_EA0_RDREQ_64B_sum"] + 128 * a["TCC_EA0_RDREQ_128B_sum"]
        wr = 32 * (b["TCC_EA0_WRREQ_sum"] - b["TCC_EA0_WRREQ_64B_sum"]) + 64 * b["TCC_EA0_WRREQ_64B_sum"]
        kernels[k] = {"dispatches": n, "read_bytes": rd, "write_bytes": wr,
                      "dram_read_bytes": 32 * b["TCC_EA0_RDREQ_DRAM_32B_sum"],
                      "fetch_size_bytes": 1024 * c.get("FETCH_SIZE", 0.0),
                      "write_size_bytes": 1024 * d.get("WRITE_SIZE", 0.0)}
    out = {"workload": workload, "kernel_source_hash": kernel_source_hash(),
           "counts": "L2-to-fabric bytes per dispatch (TCC_EA0 read requests by size, write requests); "
                     "last-level (Infinity) cache hits included, so an upper bound on HBM bytes",
           "kernels": kernels}
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
    for k, v in sorted(kernels.items(), key=lambda kv: -kv[1]["read_bytes"]):
        print(f"{k:22s} n={v['dispatches']:5d} read {v['read_bytes'] / 1e6:10.1f} MB  write {v['write_bytes'] / 1e6:9.1f} MB"
              f"  (FETCH_SIZE {v['fetch_size_bytes'] / 1e6:9.1f} MB, WRITE_SIZE {v['write_size_bytes'] / 1e6:9.1f} MB)")


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
    ap.add_argument("--tokens", type=int, default=0,
                    help="the gpt-oss head (H 2880, V 201088, K 64, tau 1) at this many tokens, as in the sweep")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-seq-chunk", action="store_true", help="skip the sequence-chunk schedule line")
    ap.add_argument("--no-variants", action="store_true", help="skip the logits / top-K variant lines")
    ap.add_argument("--cpu-rows", type=int, default=4096,
                    help="tokens of the workload the CPU oracle is timed on (default: all of the gpt-oss head's)")
    ap.add_argument("--no-scaling", action="store_true", help="skip the long / qwen / T-sweep lines")
    ap.add_argument("--summarize-counters", nargs=3, metavar=("PMC_DIR", "WORKLOAD", "OUT_JSON"),
                    help="per-kernel L2-to-fabric bytes from four rocprofv3 --pmc passes (see summarize_counters)")
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
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
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
    wl = (synth.Workload(f"sweep-T{args.tokens}", args.tokens, 2880, 201088, 64, 1.0) if args.tokens
          else synth.WORKLOADS[args.workload])
    res, x = run_one(args, wl)
    res["config"]["schedule"] = "recompute (pass 2 recomputes each vocabulary chunk)"
    if not args.no_seq_chunk:
        res["seq_chunk"] = run_seq_chunk(args, wl, x)
    if not args.no_variants:
        res["logits_variant"] = run_logits_variant(args, wl, x)
        res["topk_variant"] = res["logits_variant"].pop("topk_variant")
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(x, wl.tau, args.cpu_rows)
        res["cpu_baseline"]["tiny_full"] = cpu_tiny_full()
    else:
        res["cpu_baseline"] = None
    del x
    if not args.no_scaling and args.workload == "gptoss" and not args.tokens:
        res["scaling"] = scaling_lines(args)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
