"""The fused call captured in a HIP graph (torch.cuda.CUDAGraph on the
current stream): it launches kernels only (no memset, no allocation, no
synchronisation when validation is off), so a captured call replays to the
same loss and gradients as the eager call, bit for bit (every reduction has a
fixed order).  Each replay follows eager work on the same inputs, and every
replay is checked."""
import pytest

torch = pytest.importorskip("torch")

import chunked_kl_loss_02_amd as kd
import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seq_chunk", [False, True])
def test_fused_call_replays_in_a_graph(seq_chunk):
    print(f"[case] graph capture seq_chunk={seq_chunk}", flush=True)
    # several token blocks (the last ragged) x several vocabulary chunks (the last ragged)
    x = synth.make_inputs_torch(600, 256, 5000, 16, seed=21, mask="packed8")
    args = (x["h"], x["W"], x["teacher_idx"], x["teacher_logit"], x["mask"], 1.5)
    kw = dict(chunk_v=1024, block_t=256, seq_chunk=seq_chunk, row_loss=True)
    eager = [t.clone() for t in kd.fwd_bwd(*args, **kw)]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        kd.fwd_bwd(*args, **kw)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        captured = kd.fwd_bwd(*args, **kw)
    torch.cuda.synchronize()
    for r in range(3):
        other = kd.fwd_bwd(*args, **kw)  # eager work between replays
        torch.cuda.synchronize()
        for t in captured:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b, c in zip(("loss", "dH", "dW", "row_loss"), captured, eager, other):
            assert torch.equal(a, b), (r, name)
            assert torch.equal(c, b), (r, name)
