"""kd_topk_kl_fwd_bwd_noalloc (the library's static per-GPU scratch in place
of a caller workspace) against kd_topk_kl_fwd_bwd on the same problems:
bitwise equal loss, dH, dW and per-row loss on calls in a row, each later
one smaller (the scratch keeps the previous call's contents), and within
the oracle tolerances of the fp64 CPU oracle."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import chunked_kl_loss_02_amd as kd
import synth
from oracle import kl_dense

pytestmark = pytest.mark.gpu


def to_dev(x):
    h = torch.from_numpy(x["h_bits"].view(np.int16)).view(torch.bfloat16).cuda()
    W = torch.from_numpy(x["W_bits"].view(np.int16)).view(torch.bfloat16).cuda()
    idx = torch.from_numpy(x["teacher_idx"]).cuda()
    lg = torch.from_numpy(x["teacher_logit"]).cuda()
    m = torch.from_numpy(x["mask"]).cuda()
    return h, W, idx, lg, m


def nrel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def run_pair(h, W, idx, lg, m, tau, **kw):
    print(f"[noalloc] T={h.shape[0]} H={h.shape[1]} V={W.shape[0]} K={idx.shape[1]} tau={tau} {kw}", flush=True)
    T, H = h.shape
    V = W.shape[0]
    ref = kd.fwd_bwd(h, W, idx, lg, m, tau, row_loss=True, **kw)
    nan = float("nan")
    out = (torch.full((), nan, device="cuda"), torch.full((T, H), nan, device="cuda"),
           torch.full((V, H), nan, device="cuda"), torch.full((T,), nan, device="cuda"))
    got = kd.fwd_bwd_noalloc(h, W, idx, lg, m, tau, out=out, row_loss=True, **kw)
    torch.cuda.synchronize()
    for name, a, b in zip(("loss", "dH", "dW", "row_loss"), got, ref):
        assert torch.equal(a, b), name
    return got


def check_oracle(x, tau, got):
    ref = kl_dense(x["h"], x["W"], x["teacher_idx"], x["teacher_logit"], x["mask"], tau)
    el = abs(got[0].item() - ref["loss"]) / abs(ref["loss"])
    eh = nrel(got[1].cpu().double().numpy(), ref["dH"])
    ew = nrel(got[2].cpu().double().numpy(), ref["dW"])
    print(f"  loss rel {el:.2e} dH {eh:.2e} dW {ew:.2e}", flush=True)
    assert el <= 1e-3 and eh <= 2e-2 and ew <= 2e-2


def test_noalloc_equals_workspace_entry_point_on_calls_in_a_row():
    # 4 token blocks x 5 vocabulary chunks (both ragged), packed mask
    x1 = synth.make_inputs_np(1000, 512, 20000, 32, seed=31, mask="packed8")
    g1 = run_pair(*to_dev(x1), 1.3, chunk_v=4096, block_t=256)
    check_oracle(x1, 1.3, g1)
    # smaller: one block, one chunk, ragged tiles
    x2 = synth.make_inputs_np(300, 256, 5000, 16, seed=32)
    g2 = run_pair(*to_dev(x2), 0.8, chunk_v=8192)
    check_oracle(x2, 0.8, g2)
    # smaller still, sequence-chunk schedule
    x3 = synth.make_inputs_np(100, 128, 3000, 8, seed=33)
    run_pair(*to_dev(x3), 1.0, chunk_v=1024, seq_chunk=True)


@pytest.mark.parametrize("H", [320, 384])
def test_short_last_hidden_tile_equals_the_full_height_tile(H):
    # the workspace entry point computes the last hidden tile 64 (H = 320) or 128 (H = 384)
    # rows high, the allocation-free one at the full 256 rows: the same dot products in the
    # same k order, so bitwise the same outputs (several blocks and chunks, accumulation in both)
    x = synth.make_inputs_np(700, H, 3000, 16, seed=35, mask="packed8")
    run_pair(*to_dev(x), 0.9, chunk_v=1024, block_t=256)


def test_noalloc_gpt_oss_head_with_8192_row_chunks():
    # the documented fit: T 4096, H 2880, V 201088, K 64 at chunk_v 8192
    x = synth.make_inputs_torch(4096, 2880, 201088, 64, seed=2)
    # its single-gradient-buffer plan: the workspace less one 4096 x 8192 bf16 buffer and the copy
    # of W's last 64 columns (that plan computes the last hidden tile at full height)
    assert kd.workspace_size(4096, 2880, 201088, 64, 1.0, chunk_v=8192) - 4096 * 8192 * 2 - 64 * 201088 * 2 <= \
        kd.NOALLOC_SCRATCH_BYTES
    run_pair(x["h"], x["W"], x["teacher_idx"], x["teacher_logit"], x["mask"], 1.0, chunk_v=8192)


def test_noalloc_refuses_a_problem_beyond_its_scratch():
    x = synth.make_inputs_np(64, 64, 300, 4, seed=34)
    h, W, idx, lg, m = to_dev(x)
    out = (torch.empty((), device="cuda"), torch.empty((64, 64), device="cuda"), torch.empty((300, 64), device="cuda"))
    # a 262144-row vocabulary chunk: 256 x 262144 bf16 gradient buffer (128 MiB) plus per-token
    # state (one block and one chunk: a single buffer either way)
    assert kd.workspace_size(64, 64, 300, 4, 1.0, chunk_v=262144) > kd.NOALLOC_SCRATCH_BYTES
    with pytest.raises(kd.KdError) as e:
        kd.fwd_bwd_noalloc(h, W, idx, lg, m, 1.0, out=out, chunk_v=262144)
    assert e.value.code == 3


def test_noalloc_call_replays_in_a_graph():
    # the callers it is for: code under graph capture.  The first call on the
    # GPU resolves the scratch address, outside the capture
    print("[noalloc] graph capture", flush=True)
    x = synth.make_inputs_torch(600, 256, 5000, 16, seed=22, mask="packed8")
    args = (x["h"], x["W"], x["teacher_idx"], x["teacher_logit"], x["mask"], 1.5)
    kw = dict(chunk_v=1024, block_t=256, row_loss=True)
    out = (torch.empty((), device="cuda"), torch.empty((600, 256), device="cuda"),
           torch.empty((5000, 256), device="cuda"), torch.empty((600,), device="cuda"))
    kd.fwd_bwd_noalloc(*args, out=out, **kw)
    torch.cuda.synchronize()
    eager = [t.clone() for t in out]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kd.fwd_bwd_noalloc(*args, out=out, **kw)
    torch.cuda.synchronize()
    for r in range(3):
        other = kd.fwd_bwd(*args, **kw)  # eager work between replays
        torch.cuda.synchronize()
        for t in out:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b, c in zip(("loss", "dH", "dW", "row_loss"), out, eager, other):
            assert torch.equal(a, b), (r, name)
            assert torch.equal(c, b), (r, name)
