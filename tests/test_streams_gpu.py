"""The fused call is reentrant across streams given distinct workspaces
(include/kdkl.h): two calls enqueued on two streams at once give bitwise the
results of the same calls run one after the other."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import chunked_kl_loss_02_amd as kd
import synth

pytestmark = pytest.mark.gpu


def dev(x):
    h = torch.from_numpy(x["h_bits"].view(np.int16)).view(torch.bfloat16).cuda()
    W = torch.from_numpy(x["W_bits"].view(np.int16)).view(torch.bfloat16).cuda()
    return (h, W, torch.from_numpy(x["teacher_idx"]).cuda(), torch.from_numpy(x["teacher_logit"]).cuda(),
            torch.from_numpy(x["mask"]).cuda())


def test_two_streams_with_distinct_workspaces():
    print("[case] two streams, two problems", flush=True)
    # two different problems: several blocks and chunks each
    a = dev(synth.make_inputs_np(700, 256, 6000, 16, seed=41, mask="packed8"))
    b = dev(synth.make_inputs_np(900, 256, 6000, 16, seed=42))
    kw = dict(chunk_v=1024, block_t=256)
    ref_a = kd.fwd_bwd(*a, 1.1, **kw)
    ref_b = kd.fwd_bwd(*b, 0.9, **kw)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()  # default priority
    for _ in range(3):
        with torch.cuda.stream(s1):
            got_a = kd.fwd_bwd(*a, 1.1, **kw)
        with torch.cuda.stream(s2):
            got_b = kd.fwd_bwd(*b, 0.9, **kw)
        torch.cuda.synchronize()
        for r, g in ((ref_a, got_a), (ref_b, got_b)):
            for x, y in zip(r, g):
                assert torch.equal(x, y)
