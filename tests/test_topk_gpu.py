"""GPU tests of the per-row top-K selection (kd_topk_select) against the
oracle's topk_rows: ids and values must match exactly (the order is unique:
descending value, equal values by ascending id)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import chunked_kl_loss_02_amd as kd
import synth
from oracle import topk_rows

pytestmark = pytest.mark.gpu


def check(Xf, K):
    """Xf: float32 values, rounded to bf16 first (the kernel's input type)."""
    Xf = synth.round_bf16_np(np.ascontiguousarray(Xf, dtype=np.float32))
    T, V = Xf.shape
    print(f"[topk] T={T} V={V} K={K}", flush=True)
    X = torch.from_numpy(Xf).to("cuda").to(torch.bfloat16).contiguous()
    idx, val = kd.topk_select(X, K)
    torch.cuda.synchronize()
    ref_idx, ref_val = topk_rows(Xf, K)
    gi, gv = idx.cpu().numpy(), val.cpu().numpy()
    bad = np.nonzero(np.any(gi != ref_idx, axis=1))[0]
    assert bad.size == 0, f"rows {bad[:5]}: got {gi[bad[0]][:8]} want {ref_idx[bad[0]][:8]}"
    assert np.array_equal(gv.astype(np.float64), ref_val)


@pytest.mark.parametrize("V,K", [(4096, 64), (8800, 100), (8, 8), (2048, 1), (512, 512), (5000, 1024)])
def test_random_rows(V, K):
    r = np.random.default_rng(V + K)
    check(synth.round_bf16_np((r.standard_normal((67, V)) * 2).astype(np.float32)), K)


def test_heavy_ties_signed_zeros_and_infinities():
    r = np.random.default_rng(1)
    X = r.integers(-3, 4, size=(40, 2048)).astype(np.float32)   # ~290 copies of each value per row
    X[0] = 1.0                                                   # one value everywhere
    X[1, ::2] = -0.0                                              # -0 and +0 tie
    X[1, 1::2] = 0.0
    X[2, 100:110] = np.inf
    X[3] = -np.inf
    X[3, 77] = -1e30
    check(X, 100)
    check(X, 1)


def test_teacher_rows_at_the_gpt_oss_vocabulary():
    """Rows of V = 201088 bf16 logits (the shape of the pages' teacher cache
    with K = 64 and K = 100)."""
    r = np.random.default_rng(2)
    X = synth.round_bf16_np((r.standard_normal((48, 201088)) * 2).astype(np.float32))
    check(X, 64)
    check(X, 100)


def test_top_values_crowded_into_one_threads_share():
    """A row's 512 threads each keep their two best elements from one pass;
    a thread holding more of the top K (here all of them, or pairs of equal
    values) must rescan its share.  Thread r's share is vectors r, r + 512, ...
    of 8 values each."""
    r = np.random.default_rng(4)
    V = 201088
    X = (r.standard_normal((6, V)) * 2).astype(np.float32)
    share = lambda tid, n: (8 * (tid + 512 * np.arange(n))[:, None] + np.arange(8)[None, :]).ravel()
    X[0, share(5, 16)[:128]] = 50.0 + np.arange(128)          # top 128 all in thread 5
    X[1, share(9, 8)[:64]] = 40.0                              # 64 equal maxima in thread 9
    X[2, share(0, 49)[-8:]] = 30.0                             # at the end of thread 0's share
    X[3, share(511, 4)] = 20.0 + np.arange(32) % 3             # ties inside one thread
    check(X, 64)
    check(X, 100)


def test_unsupported_shapes_are_rejected():
    X = torch.zeros(4, 1001, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kd.KdError) as e:
        kd.topk_select(X, 4)
    assert e.value.code == 2
    with pytest.raises(kd.KdError) as e:
        kd.topk_select(torch.zeros(4, 1000, dtype=torch.bfloat16, device="cuda"), 2000)
    assert e.value.code == 1


def test_long_runs_of_equal_values_take_the_exact_path():
    """More than 4096 keys at the candidate threshold (the LDS capacity): the
    kernel's exact bit-by-bit path."""
    r = np.random.default_rng(3)
    X = r.integers(-3, 4, size=(12, 16384)).astype(np.float32)
    X[0] = 2.5                      # 16384 equal values
    X[1, :9000] = 3.0               # 9000 copies of the maximum
    X[2, 5000:] = 7.0
    check(X, 64)
    check(X, 1000)
