"""Numbers the pages print, checked against the oracle's formulas and the bench's reporting."""
import json
import os

import bench

HERE = os.path.dirname(os.path.abspath(__file__))


def test_dense_teacher_tensor_size_matches_the_blog():
    g = json.load(open(os.path.join(HERE, "golden", "blog_dense_teacher_tensor.json")))
    B, V, T = g["shape"]
    n = bench.naive_logit_bytes(B * T, V, g["bytes_per_element"])
    assert n == 4 * 201088 * 32768 * 2
    # "about 50 GB": 52.7e9 bytes = 49.1 GiB
    assert abs(n / 1e9 - g["stated_gigabytes_approx"]) / g["stated_gigabytes_approx"] < 0.06
    assert abs(n / 2**30 - g["stated_gigabytes_approx"]) / g["stated_gigabytes_approx"] < 0.06


def test_flops_per_token():
    # pass-1 GEMM, pass-2 recompute, dH and dW: 2*H*V each
    assert bench.flops_per_token(2880, 201088) == 8 * 2880 * 201088
    assert abs(bench.flops_per_token(2880, 201088) / 1e9 - 4.633) < 1e-3


def test_per_kernel_flops_add_up_to_the_step():
    # the bench's per-kernel MFMA rates split 8 T H V over the library's own units: pass 1,
    # the first unit's pass 2, the merged launches, the last unit's contractions (or, with one
    # gradient buffer, every unit's pass 2 and contractions)
    for T, H, V, K in ((4096, 2880, 201088, 64), (16384, 2880, 201088, 64), (1000, 256, 4096, 32),
                       (700, 128, 3000, 16)):
        f = bench.kernel_flops(T, H, V, K, 1.0)
        assert abs(sum(f.values()) - 8.0 * T * H * V) <= 1e-9 * 8.0 * T * H * V, (T, f)
        assert f["pass1"] == 2.0 * T * H * V
