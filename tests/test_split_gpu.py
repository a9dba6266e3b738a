"""GPU tests of the split entry points (kd_topk_kl_fwd / kd_topk_kl_bwd), the
gradient flags (accumulate, bf16 outputs, an incoming gradient scale) and
the torch autograd wrapper, through the C ABI.

The split path runs the same kernels in the same order as the fused call,
so its outputs must equal the fused call's bit for bit; scaled gradients and
the autograd path are also checked against the fp64 oracle with the parity
tolerances (dH, dW normwise relative error <= 2e-2)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import chunked_kl_loss_02_amd as kd
import synth
from oracle import kl_dense

pytestmark = pytest.mark.gpu

GRAD_TOL = 2e-2


def nrel(a, b):
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a))


def inputs(T, H, V, K, seed, masked=()):
    x = synth.make_inputs_np(T, H, V, K, seed=seed)
    x["mask"][list(masked)] = 0
    dev = "cuda"
    h = torch.from_numpy(x["h_bits"].view(np.int16)).view(torch.bfloat16).to(dev)
    W = torch.from_numpy(x["W_bits"].view(np.int16)).view(torch.bfloat16).to(dev)
    idx = torch.from_numpy(np.ascontiguousarray(x["teacher_idx"], dtype=np.int32)).to(dev)
    lg = torch.from_numpy(np.ascontiguousarray(x["teacher_logit"], dtype=np.float32)).to(dev)
    m = torch.from_numpy(np.ascontiguousarray(x["mask"], dtype=np.uint8)).to(dev)
    return x, (h, W, idx, lg, m)


# ragged in every dimension, several token blocks and vocabulary chunks
CASE = dict(T=600, H=192, V=4261, K=100, seed=21, masked=(3, 50, 599))
KW = dict(chunk_v=1024, block_t=256)
TAU = 2.0


def test_split_equals_fused_bitwise():
    print("[split] fwd + bwd vs fwd_bwd", flush=True)
    x, (h, W, idx, lg, m) = inputs(**CASE)
    loss0, dH0, dW0, rl0, ws = kd.fwd_bwd(h, W, idx, lg, m, TAU, row_loss=True, return_workspace=True, **KW)
    loss1, saved, rl1 = kd.fwd(h, W, idx, lg, m, TAU, row_loss=True, **KW)
    dH1, dW1 = kd.bwd(saved, h, W, idx, lg, m, TAU, **KW)
    # the saved state is only read: a second backward gives the same bits
    dH2, dW2 = kd.bwd(saved, h, W, idx, lg, m, TAU, **KW)
    torch.cuda.synchronize()
    assert torch.equal(loss0, loss1)
    assert torch.equal(rl0, rl1)
    assert torch.equal(dH0, dH1) and torch.equal(dW0, dW1)
    assert torch.equal(dH1, dH2) and torch.equal(dW1, dW2)
    T = CASE["T"]
    assert torch.equal(kd.saved_lse(saved, T), kd.lse(ws, T, CASE["H"], CASE["V"], CASE["K"], TAU, **KW))
    ref = kl_dense(x["h"], x["W"], x["teacher_idx"], x["teacher_logit"], x["mask"], TAU)
    assert abs(loss1.item() - ref["loss"]) <= 1e-3 * abs(ref["loss"])
    assert np.max(np.abs(kd.saved_lse(saved, T).cpu().double().numpy() - ref["lse"])) <= 1e-3


def test_split_backward_ignores_the_sequence_chunk_flag():
    # through the C ABI: kd_topk_kl_bwd with KD_FLAG_SEQ_CHUNK set equals the call without it,
    # bit for bit, with a workspace sized for the problem without the flag
    print("[split] bwd with the sequence-chunk flag", flush=True)
    import ctypes
    x, (h, W, idx, lg, m) = inputs(**CASE)
    T, H, V, K = CASE["T"], CASE["H"], CASE["V"], CASE["K"]
    _, saved = kd.fwd(h, W, idx, lg, m, TAU, **KW)
    dH0, dW0 = kd.bwd(saved, h, W, idx, lg, m, TAU, **KW)
    p = kd.problem(T, H, V, K, TAU, KW["chunk_v"], KW["block_t"], flags=kd.KD_FLAG_SEQ_CHUNK)
    ws = torch.empty(kd.workspace_size(T, H, V, K, TAU, **KW), dtype=torch.uint8, device="cuda")
    dH1 = torch.empty_like(dH0)
    dW1 = torch.empty_like(dW0)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    code = kd.lib().kd_topk_kl_bwd(ctypes.byref(p), ptr(h), ptr(W), ptr(idx), ptr(lg), ptr(m), ptr(saved),
                                   ctypes.c_void_p(0), ptr(dH1), ptr(dW1), ptr(ws), ctypes.c_size_t(ws.numel()),
                                   stream)
    torch.cuda.synchronize()
    assert code == 0
    assert torch.equal(dH0, dH1) and torch.equal(dW0, dW1)


@pytest.mark.parametrize("g", [-2.5, 0.0, 1e-3])
def test_incoming_gradient_scales_the_backward(g):
    print(f"[split] grad_loss = {g}", flush=True)
    x, (h, W, idx, lg, m) = inputs(**CASE)
    _, saved = kd.fwd(h, W, idx, lg, m, TAU, **KW)
    gl = torch.tensor(g, dtype=torch.float32, device="cuda")
    dH, dW = kd.bwd(saved, h, W, idx, lg, m, TAU, grad_loss=gl, **KW)
    torch.cuda.synchronize()
    ref = kl_dense(x["h"], x["W"], x["teacher_idx"], x["teacher_logit"], x["mask"], TAU)
    if g == 0.0:
        assert not torch.any(dH).item() and not torch.any(dW).item()
        return
    eh = nrel(dH.double().cpu().numpy(), g * ref["dH"])
    ew = nrel(dW.double().cpu().numpy(), g * ref["dW"])
    print(f"  dH {eh:.2e} dW {ew:.2e}", flush=True)
    assert eh <= GRAD_TOL and ew <= GRAD_TOL


def test_accumulate_and_bf16_outputs():
    print("[split] accumulate / bf16", flush=True)
    x, (h, W, idx, lg, m) = inputs(**CASE)
    T, H, V = CASE["T"], CASE["H"], CASE["V"]
    _, saved = kd.fwd(h, W, idx, lg, m, TAU, **KW)
    dH, dW = kd.bwd(saved, h, W, idx, lg, m, TAU, **KW)
    gen = torch.Generator(device="cuda").manual_seed(5)
    base_h = torch.randn(T, H, device="cuda", generator=gen)
    base_w = torch.randn(V, H, device="cuda", generator=gen)
    # fp32 accumulate: the contraction adds onto the existing values
    aH, aW = base_h.clone(), base_w.clone()
    kd.bwd(saved, h, W, idx, lg, m, TAU, dH=aH, dW=aW, accumulate_dh=True, accumulate_dw=True, **KW)
    # bf16 outputs: one rounding of the same fp32 result
    bH, bW = kd.bwd(saved, h, W, idx, lg, m, TAU, grad_dtype=torch.bfloat16, **KW)
    # bf16 accumulate: one rounding of (previous bf16 value + fp32 result)
    cH, cW = base_h.to(torch.bfloat16), base_w.to(torch.bfloat16)
    pH, pW = cH.clone(), cW.clone()
    kd.bwd(saved, h, W, idx, lg, m, TAU, dH=cH, dW=cW, accumulate_dh=True, accumulate_dw=True, **KW)
    # fused call with bf16 outputs
    _, fH, fW = kd.fwd_bwd(h, W, idx, lg, m, TAU, grad_dtype=torch.bfloat16, **KW)
    torch.cuda.synchronize()
    # the same sum in another order: a few fp32 roundings of values of size |base| <= ~6
    assert torch.allclose(aH, base_h + dH, rtol=0, atol=1e-5)
    assert torch.allclose(aW, base_w + dW, rtol=0, atol=1e-5)
    assert bH.dtype == torch.bfloat16 and bW.dtype == torch.bfloat16
    assert torch.equal(bH, dH.to(torch.bfloat16)) and torch.equal(bW, dW.to(torch.bfloat16))
    assert torch.equal(fH, bH) and torch.equal(fW, bW)
    assert torch.equal(cH, (pH.float() + dH).to(torch.bfloat16))
    assert torch.equal(cW, (pW.float() + dW).to(torch.bfloat16))


def test_autograd_function():
    print("[split] autograd", flush=True)
    x, (h, W, idx, lg, m) = inputs(**CASE)
    hh = h.clone().requires_grad_(True)
    WW = W.clone().requires_grad_(True)
    loss = kd.topk_kl_loss(hh, WW, idx, lg, m, TAU, **KW)
    (3.0 * loss).backward()
    torch.cuda.synchronize()
    assert hh.grad.dtype == torch.bfloat16 and WW.grad.dtype == torch.bfloat16
    ref = kl_dense(x["h"], x["W"], x["teacher_idx"], x["teacher_logit"], x["mask"], TAU)
    assert abs(loss.item() - ref["loss"]) <= 1e-3 * abs(ref["loss"])
    eh = nrel(hh.grad.double().cpu().numpy(), 3.0 * ref["dH"])
    ew = nrel(WW.grad.double().cpu().numpy(), 3.0 * ref["dW"])
    print(f"  dH {eh:.2e} dW {ew:.2e}", flush=True)
    assert eh <= GRAD_TOL and ew <= GRAD_TOL
    # only the requested gradient is formed
    hh2 = h.clone().requires_grad_(True)
    kd.topk_kl_loss(hh2, W, idx, lg, None, TAU, **KW).backward()
    assert hh2.grad is not None and torch.all(torch.isfinite(hh2.grad.float())).item()


def test_split_empty_batch():
    print("[split] T = 0", flush=True)
    H, V, K = 128, 1000, 8
    h = torch.empty(0, H, dtype=torch.bfloat16, device="cuda")
    W = torch.randn(V, H, device="cuda").to(torch.bfloat16)
    idx = torch.empty(0, K, dtype=torch.int32, device="cuda")
    lg = torch.empty(0, K, dtype=torch.float32, device="cuda")
    loss, saved = kd.fwd(h, W, idx, lg, None, 1.0)
    dW = torch.full((V, H), 7.0, device="cuda")
    kd.bwd(saved, h, W, idx, lg, None, 1.0, grad_h=False, dW=dW)
    torch.cuda.synchronize()
    assert loss.item() == 0.0
    assert not torch.any(dW).item()
