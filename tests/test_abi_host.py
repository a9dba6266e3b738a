"""C-ABI checks that need the built library but no GPU: every function that
include/kdkl.h declares is exported, the workspace planner, and argument
validation (which returns before any HIP call)."""
import ctypes
import os
import re
import subprocess

import pytest

import chunked_kl_loss_02_amd as kd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kdkl.h")

pytestmark = pytest.mark.skipif(not os.path.exists(kd.library_path),
                                reason="libkdkl.so not built (run __graft_entry__.build())")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kd_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("kd_topk_kl_fwd_bwd", "kd_topk_kl_workspace_size", "kd_status_string", "kd_topk_kl_fwd",
              "kd_topk_kl_bwd", "kd_topk_kl_saved_size", "kd_topk_kl_fwd_workspace_size"):
        assert n in names


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", kd.library_path], capture_output=True, text=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if l.strip())
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    L = kd.lib()
    for n in declared_functions():
        assert hasattr(L, n)
    assert L.kd_abi_version() == kd.ABI_VERSION == 5


def _ws(T, H, V, K, tau=1.0, chunk_v=0, block_t=0):
    p = kd.problem(T, H, V, K, tau, chunk_v, block_t)
    n = ctypes.c_size_t(0)
    code = kd.lib().kd_topk_kl_workspace_size(ctypes.byref(p), ctypes.byref(n))
    return code, n.value


def test_workspace_plan():
    code, n = _ws(4096, 2880, 201088, 64)
    assert code == 0
    # two gradient buffers (4096 x 12288 bf16: one unit's contractions run
    # beside the next unit's pass 2), the block's h^T (2880 x 4096 bf16), the
    # k-contiguous copy of W's last 64 columns (2880 = 11 x 256 + 64: the last
    # hidden tile of the contractions is 64 rows high) plus per-token state
    fixed = 2 * 4096 * 12288 * 2 + 2880 * 4096 * 2 + 64 * 201088 * 2
    assert fixed <= n < fixed + 4096 * 8 * 1024
    # per-token growth is linear once T exceeds one block
    _, a = _ws(65536, 2880, 201088, 64)
    _, b = _ws(131072, 2880, 201088, 64)
    _, c = _ws(262144, 2880, 201088, 64)
    assert abs((c - b) - 2 * (b - a)) <= 4096
    # bytes per token of workspace (teacher probabilities, merged mass, gathered
    # logit, bucketed entry and its index: 5 K words, plus a few per-token
    # scalars and the per-tile bucket counts), far below one bf16 logit row
    # (2V = 402 KB)
    assert (c - b) / 131072 < 20 * 64 + 64


@pytest.mark.parametrize("args,code", [
    ((4096, 2880, 201088, 64, 0.0), 1),          # tau <= 0
    ((4096, 2880, 201088, 64, float("nan")), 1),
    ((4096, 2880, 201088, 64, float("inf")), 1),
    ((4096, 2880, 201088, 0, 1.0), 1),           # K = 0
    ((4096, 2880, 50, 64, 1.0), 1),              # K > V
    ((-1, 2880, 201088, 64, 1.0), 1),            # T < 0
    ((4096, 2900, 201088, 64, 1.0), 2),          # H % 64
    ((4096, 2880, 201088, 2000, 1.0), 2),        # K > 1024
    ((0, 2880, 201088, 64, 1.0), 0),             # T = 0 is fine
])
def test_workspace_size_validation(args, code):
    assert _ws(*args)[0] == code


def test_chunk_and_block_must_be_multiples_of_256():
    assert _ws(1000, 128, 5000, 8, 1.0, 300, 0)[0] == 2
    assert _ws(1000, 128, 5000, 8, 1.0, 0, 100)[0] == 2
    assert _ws(1000, 128, 5000, 8, 1.0, 512, 768)[0] == 0


def test_fp32_gradient_targets_must_fit_32_bit_offsets():
    """The gradient contractions read back and add to fp32 dH / dW rows of
    one token block / vocabulary chunk through 32-bit byte offsets, so
    chunk * H * 4 and block * H * 4 must stay below 4 GiB; a problem over
    that is refused instead of wrapping."""
    # 12288-row chunk x H = 98304: 2.4 GB of bf16 W rows (under 4 GiB) but
    # 4.8 GB of fp32 dW rows
    assert _ws(4096, 98304, 201088, 64)[0] == 2
    assert _ws(4096, 98304, 201088, 64, 1.0, 12288, 0)[0] == 2
    assert _ws(4096, 98304, 201088, 64, 1.0, 8192, 0)[0] == 0
    # one chunk spanning a 262144-token vocabulary at H = 5120 (5.4 GB fp32)
    assert _ws(512, 5120, 262144, 64, 1.0, 262144, 256)[0] == 2
    assert _ws(512, 5120, 262144, 64, 1.0, 131072, 256)[0] == 0
    # a token block of 16384 at H = 65536 (4.3 GB of fp32 dH rows)
    assert _ws(65536, 65536, 4096, 8, 1.0, 256, 16384)[0] == 2
    assert _ws(65536, 65536, 4096, 8, 1.0, 256, 8192)[0] == 0
    # the same bound holds for the split backward and the forward sizes
    L = kd.lib()
    assert _size(L.kd_topk_kl_fwd_workspace_size, 512, 5120, 262144, 64, chunk_v=262144, block_t=256)[0] == 2


def test_stored_logit_rows_of_a_block_must_fit_32_bit_offsets():
    """The sequence-chunk schedule's gradient tiles read 256 stored fp32
    logit rows of a token block (one column per token) through one 32-bit
    buffer range, so 256 * block * 4 bytes must stay below 4 GiB."""
    def ws(block_t, flags):
        p = kd.problem(block_t, 64, 1000, 1, 1.0, 256, block_t, flags=flags)
        n = ctypes.c_size_t(0)
        return kd.lib().kd_topk_kl_workspace_size(ctypes.byref(p), ctypes.byref(n))
    assert ws(4194304, kd.KD_FLAG_SEQ_CHUNK) == 2          # exactly 4 GiB
    assert ws(4194304 - 256, kd.KD_FLAG_SEQ_CHUNK) == 0
    assert ws(4194304, 0) == 0                             # the recompute schedule stores none


def test_launch_grids_stay_under_2_to_the_32_work_items():
    """A dispatch holds at most 2^32 - 1 work-items: the per-token teacher
    kernel (64 per token), the per-entry bucket kernels (one per entry) and
    pass 1 (256 per token tile x vocabulary tile of a block) bound T, T * K
    and block * V; a problem past them is refused instead of failing at
    launch."""
    assert _ws((1 << 26) - 256, 64, 1000, 1)[0] == 0
    assert _ws((1 << 26) - 255, 64, 1000, 1)[0] == 2
    assert _ws(1 << 22, 64, 2048, 1023)[0] == 0            # T K = 2^32 - 2^22
    assert _ws(1 << 22, 64, 2048, 1024)[0] == 2            # T K = 2^32
    # pass 1 over 32 token tiles x 2^19 vocabulary tiles (2^24 tiles) ...
    assert _ws(8192, 64, 1 << 27, 1, 1.0, 0, 8192)[0] == 2
    # ... or over one token tile: fine
    assert _ws(256, 64, 1 << 27, 1, 1.0, 0, 256)[0] == 0
    assert _ws(8192, 64, 1 << 24, 1, 1.0, 0, 8192)[0] == 0
    L = kd.lib()
    n = ctypes.c_size_t(0)
    ok = kd.KdLogitsProblem((1 << 23) - 1, 1000, 4, 1.0, 0)
    assert L.kd_topk_kl_logits_workspace_size(ctypes.byref(ok), ctypes.byref(n)) == 0
    big = kd.KdLogitsProblem(1 << 23, 1000, 4, 1.0, 0)
    assert L.kd_topk_kl_logits_workspace_size(ctypes.byref(big), ctypes.byref(n)) == 2


def test_fwd_bwd_rejects_bad_arguments_before_any_hip_call():
    L = kd.lib()
    vp = ctypes.c_void_p
    p = kd.problem(16, 64, 100, 4)
    fake = vp(1 << 20)  # never dereferenced: validation fails first
    # null W
    assert L.kd_topk_kl_fwd_bwd(ctypes.byref(p), fake, vp(0), fake, fake, vp(0), fake, vp(0), vp(0), vp(0),
                                fake, ctypes.c_size_t(1 << 30), vp(0)) == 1
    # misaligned h
    assert L.kd_topk_kl_fwd_bwd(ctypes.byref(p), vp((1 << 20) + 2), fake, fake, fake, vp(0), fake, vp(0), vp(0),
                                vp(0), fake, ctypes.c_size_t(1 << 30), vp(0)) == 2
    # workspace too small
    assert L.kd_topk_kl_fwd_bwd(ctypes.byref(p), fake, fake, fake, fake, vp(0), fake, vp(0), vp(0), vp(0),
                                fake, ctypes.c_size_t(16), vp(0)) == 3
    # bad problem
    bad = kd.problem(16, 64, 100, 4, tau=-1.0)
    assert L.kd_topk_kl_fwd_bwd(ctypes.byref(bad), fake, fake, fake, fake, vp(0), fake, vp(0), vp(0), vp(0),
                                fake, ctypes.c_size_t(1 << 30), vp(0)) == 1


def test_status_strings():
    L = kd.lib()
    for c in range(7):
        assert L.kd_status_string(c)
    assert b"workspace" in L.kd_status_string(3)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(kd, "_lib", None)
    monkeypatch.setattr(kd, "library_path", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError):
        kd.lib()


def _size(fn, T, H, V, K, flags=0, chunk_v=0, block_t=0):
    p = kd.problem(T, H, V, K, 1.0, chunk_v, block_t, flags=flags)
    n = ctypes.c_size_t(0)
    code = fn(ctypes.byref(p), ctypes.byref(n))
    return code, n.value


def test_split_entry_point_sizes():
    L = kd.lib()
    T, H, V, K = 4096, 2880, 201088, 64
    code, full = _size(L.kd_topk_kl_workspace_size, T, H, V, K)
    assert code == 0
    code, fwd = _size(L.kd_topk_kl_fwd_workspace_size, T, H, V, K)
    assert code == 0
    # the forward needs no gradient buffers (2 x 4096 x 12288 bf16), no h^T (2880 x 4096 bf16),
    # no copy of W's last 64 columns (64 x 201088 bf16) and no per-token pass-2 offsets
    # (4096 fp32); both bucket the teacher entries by tile
    assert full - fwd == 2 * 4096 * 12288 * 2 + H * 4096 * 2 + 64 * V * 2 + 4 * 4096
    code, saved = _size(L.kd_topk_kl_saved_size, T, H, V, K)
    assert code == 0
    # log-sum-exp [T] and the gathered logits [T, K], fp32, 256-byte aligned pieces
    assert 4 * T + 4 * T * K <= saved <= 4 * T + 4 * T * K + 1024
    # bf16 gradient outputs stage fp32 dH [T, H] and one dW chunk [12288, H]
    code, b16 = _size(L.kd_topk_kl_workspace_size, T, H, V, K, flags=kd.KD_FLAG_GRAD_BF16)
    assert code == 0
    assert b16 - full == 4 * T * H + 4 * 12288 * H
    # accumulate flags change nothing in the plan; unknown flags are rejected
    assert _size(L.kd_topk_kl_workspace_size, T, H, V, K,
                 flags=kd.KD_FLAG_ACCUMULATE_DH | kd.KD_FLAG_ACCUMULATE_DW) == (0, full)
    assert _size(L.kd_topk_kl_workspace_size, T, H, V, K, flags=32)[0] == 1
    # the sequence-chunk schedule keeps one token block of fp32 logits (block 4096 by default)
    # and two gradient buffers (one chunk's contractions run beside the next chunk's gradient
    # tiles), of vocabulary chunks of 16384 by default (12288 otherwise)
    code, sq = _size(L.kd_topk_kl_workspace_size, T, H, V, K, flags=kd.KD_FLAG_SEQ_CHUNK)
    assert code == 0 and sq - full == 4 * V * 4096 + 2 * 4096 * 16384 * 2 - 2 * 4096 * 12288 * 2
    # at equal tiling both schedules keep two gradient buffers: they differ by the block's logits
    assert _size(L.kd_topk_kl_workspace_size, T, H, V, K, flags=kd.KD_FLAG_SEQ_CHUNK, block_t=1024,
                 chunk_v=12288)[1] - _size(L.kd_topk_kl_workspace_size, T, H, V, K, block_t=1024)[1] == \
        4 * V * 1024
    for fn in (L.kd_topk_kl_saved_size, L.kd_topk_kl_fwd_workspace_size):
        assert _size(fn, T, 2900, V, K)[0] == 2


def test_split_entry_points_reject_bad_arguments_before_any_hip_call():
    L = kd.lib()
    vp = ctypes.c_void_p
    p = kd.problem(16, 64, 100, 4)
    fake = vp(1 << 20)
    big = ctypes.c_size_t(1 << 30)
    # fwd: null saved, misaligned saved, small workspace
    assert L.kd_topk_kl_fwd(ctypes.byref(p), fake, fake, fake, fake, vp(0), fake, vp(0), vp(0), fake, big,
                            vp(0)) == 1
    assert L.kd_topk_kl_fwd(ctypes.byref(p), fake, fake, fake, fake, vp(0), fake, vp(0), vp((1 << 20) + 16), fake,
                            big, vp(0)) == 2
    assert L.kd_topk_kl_fwd(ctypes.byref(p), fake, fake, fake, fake, vp(0), fake, vp(0), fake, fake,
                            ctypes.c_size_t(8), vp(0)) == 3
    # bwd: null saved, misaligned dH, small workspace
    assert L.kd_topk_kl_bwd(ctypes.byref(p), fake, fake, fake, fake, vp(0), vp(0), vp(0), fake, vp(0), fake, big,
                            vp(0)) == 1
    assert L.kd_topk_kl_bwd(ctypes.byref(p), fake, fake, fake, fake, vp(0), fake, vp(0), vp((1 << 20) + 4), vp(0),
                            fake, big, vp(0)) == 2
    assert L.kd_topk_kl_bwd(ctypes.byref(p), fake, fake, fake, fake, vp(0), fake, vp(0), fake, vp(0), fake,
                            ctypes.c_size_t(8), vp(0)) == 3


def test_topk_select_validates_before_any_hip_call():
    L = kd.lib()
    vp = ctypes.c_void_p
    fake = vp(1 << 20)  # never dereferenced: validation fails first

    def call(T, V, K, flags=0, X=fake):
        p = kd.KdTopkProblem(T, V, K, flags)
        return L.kd_topk_select(ctypes.byref(p), X, fake, fake, vp(0))

    assert call(4, 1000, 0) == 1               # K = 0
    assert call(4, 1000, 2000) == 1            # K > V
    assert call(4, 1000, 4, flags=1) == 1      # unknown flag
    assert call(4, 1000, 4, X=vp(0)) == 1      # null input
    assert call(4, 1001, 4) == 2               # V % 8
    assert call(4, 2048, 1025) == 2            # K > 1024
    assert call(4, 1 << 30, 4) == 2            # V past 2^30 - 1
    assert call(1 << 23, 1000, 4) == 2         # 512 work-items a row: past 2^32
    assert call(4, 1000, 4, X=vp((1 << 20) + 2)) == 2  # misaligned rows


def test_default_tiling():
    """Defaults: token blocks of 8192 (4096 for the sequence-chunk schedule),
    vocabulary chunks of 12288 while a block holds at most 4096 tokens, else
    8192 (16384 for the sequence-chunk schedule)."""
    H, V, K = 2880, 201088, 64
    for T, cv, bt in [(4096, 12288, 8192), (3000, 12288, 8192), (6000, 8192, 8192), (65536, 8192, 8192)]:
        assert _ws(T, H, V, K)[1] == _ws(T, H, V, K, chunk_v=cv, block_t=bt)[1], T
    assert _ws(65536, H, V, K)[1] != _ws(65536, H, V, K, chunk_v=12288, block_t=16384)[1]
    L = kd.lib()
    seq = kd.KD_FLAG_SEQ_CHUNK
    assert _size(L.kd_topk_kl_workspace_size, 65536, H, V, K, flags=seq)[1] == \
        _size(L.kd_topk_kl_workspace_size, 65536, H, V, K, flags=seq, chunk_v=16384, block_t=4096)[1]


def test_noalloc_rejects_problems_beyond_its_scratch_before_any_hip_call():
    L = kd.lib()
    vp = ctypes.c_void_p
    fake = vp(1 << 20)  # never dereferenced: validation fails first
    # the gpt-oss head at the default 12288-row chunk needs 146 MiB > 128 MiB
    p = kd.problem(4096, 2880, 201088, 64)
    assert _ws(4096, 2880, 201088, 64)[1] > kd.NOALLOC_SCRATCH_BYTES
    assert L.kd_topk_kl_fwd_bwd_noalloc(ctypes.byref(p), fake, fake, fake, fake, vp(0), fake, fake, fake,
                                        vp(0), vp(0)) == 3
    # with 8192-row chunks its single-buffer plan (one 4096 x 8192 bf16 gradient buffer and the
    # copy of W's last 64 columns less than kd_topk_kl_workspace_size) fits (checked on the GPU);
    # argument errors come first
    assert _ws(4096, 2880, 201088, 64, 1.0, 8192, 0)[1] - 4096 * 8192 * 2 - 64 * 201088 * 2 <= \
        kd.NOALLOC_SCRATCH_BYTES
    assert L.kd_topk_kl_fwd_bwd_noalloc(ctypes.byref(p), fake, vp(0), fake, fake, vp(0), fake, fake, fake,
                                        vp(0), vp(0)) == 1
    bad = kd.problem(16, 64, 100, 4, tau=0.0)
    assert L.kd_topk_kl_fwd_bwd_noalloc(ctypes.byref(bad), fake, fake, fake, fake, vp(0), fake, fake, fake,
                                        vp(0), vp(0)) == 1


def test_tiling_query_reports_the_default_plan():
    # one token block: 12288-row chunks, two gradient buffers (several units)
    assert kd.tiling(4096, 2880, 201088, 64) == (4096, 12288, 2)
    # blocks of 8192 above 4096 tokens take 8192-row chunks
    assert kd.tiling(16384, 2880, 201088, 64) == (8192, 8192, 2)
    # T below one block: the block is T rounded up to 256
    assert kd.tiling(1000, 2880, 201088, 64) == (1024, 12288, 2)
    # a single (block, chunk) unit needs one buffer
    assert kd.tiling(1000, 256, 4096, 32, chunk_v=4096) == (1024, 4096, 1)
    # the sequence-chunk schedule: blocks of 4096, chunks of 16384, two buffers when a block has
    # several chunks, one when the vocabulary is a single chunk
    assert kd.tiling(16384, 2880, 201088, 64, seq_chunk=True) == (4096, 16384, 2)
    assert kd.tiling(16384, 256, 16384, 32, seq_chunk=True) == (4096, 16384, 1)
    # the caller's tiling wins
    assert kd.tiling(16384, 2880, 201088, 64, chunk_v=4096, block_t=2048) == (2048, 4096, 2)


def test_binding_refuses_a_workspace_it_cannot_hand_to_the_library():
    # a workspace on another device, of another dtype or non-contiguous raises
    # before any call (its address would otherwise reach the kernels)
    torch = pytest.importorskip("torch")
    gpu = torch.device("cuda", 0)
    with pytest.raises(ValueError):
        kd._workspace(torch.empty(1024, dtype=torch.uint8), 512, gpu)
    with pytest.raises(ValueError):
        kd._workspace(torch.empty(1024, dtype=torch.float32), 512, torch.device("cpu"))
    with pytest.raises(ValueError):
        kd._workspace(torch.empty(2048, dtype=torch.uint8)[::2], 512, torch.device("cpu"))
    ws = torch.empty(1024, dtype=torch.uint8)
    assert kd._workspace(ws, 512, torch.device("cpu")) is ws
