"""Seeded input generators: bf16 rounding (checked against torch's RNE
conversion), mask recipes, teacher top-K structure and determinism."""
import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(0)
    x = np.concatenate([r.standard_normal(100000).astype(np.float32) * 3,
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5e-3, 65504.0, 0.0],
                                 np.float32)])
    ours = synth.bf16_bits_np(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(synth.round_bf16_np(x),
                          torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_masks():
    assert synth.make_mask_np(1000, "ones", 0).sum() == 1000
    m = synth.make_mask_np(32768, "packed8", 3)
    assert m[0] == 0 and (m == 0).sum() == 8
    m = synth.make_mask_np(16384, "pad10", 3)
    assert (m == 0).sum() == 1638


def test_inputs_structure_and_determinism():
    a = synth.make_inputs_np(16, 64, 500, 12, seed=5)
    b = synth.make_inputs_np(16, 64, 500, 12, seed=5)
    for k in a:
        assert np.array_equal(a[k], b[k])
    idx, val = a["teacher_idx"], a["teacher_logit"]
    assert idx.dtype == np.int32 and val.dtype == np.float32
    assert all(len(set(row.tolist())) == 12 for row in idx)
    assert np.all(np.diff(val, axis=1) <= 0)
    assert np.all((idx >= 0) & (idx < 500))
    # the bit patterns decode to the rounded float values
    assert np.array_equal((a["h_bits"].astype(np.uint32) << 16).view(np.float32), a["h"])
    # student logits have std ~ 2
    S = a["h"] @ a["W"].T
    assert 1.5 < S.std() < 2.5
