"""Seeded input generators (no GPU)."""
import numpy as np
import pytest

import workloads as W


def test_bf16_rne_hand_picked():
    f = np.array([
        1.0,                      # exact
        1.0 + 2.0**-8,            # halfway between 1.0 and 1+2^-7 -> even (1.0)
        1.0 + 3 * 2.0**-8,        # halfway between 1+2^-7 and 1+2^-6 -> even (1+2^-6)
        1.0 + 2.0**-8 + 2.0**-20, # just above halfway -> up
        -2.5,                     # exact
        3.0e38,                   # large finite
        1e-40,                    # float32 subnormal
        0.0, -0.0,
    ], dtype=np.float32)
    bits = W.f32_to_bf16_bits(f)
    assert bits.tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020,
                             0x7F62, 0x0001, 0x0000, 0x8000]


def test_bf16_matches_torch_conversion():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    ours = W.f32_to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, theirs)
    back = W.bf16_bits_to_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_dense_is_deterministic_and_shaped():
    a = W.make_dense(2, 5, 3, 8, seed=9)
    b = W.make_dense(2, 5, 3, 8, seed=9)
    for x, y in zip(a, b):
        assert x.dtype == np.uint16 and x.shape == (2, 5, 3, 8)
        np.testing.assert_array_equal(x, y)
    c = W.make_dense(2, 5, 3, 8, seed=10)
    assert not np.array_equal(a[0], c[0])


def test_rms_normalised_rows():
    q, k, v = W.make_dense(1, 50, 2, 128, seed=3, rms_qk=True)
    for x in (q, k):
        ms = np.mean(W.bf16_bits_to_f32(x).astype(np.float64) ** 2, axis=-1)
        np.testing.assert_allclose(ms, 1.0, atol=2e-2)
    msv = np.mean(W.bf16_bits_to_f32(v).astype(np.float64) ** 2, axis=-1)
    assert np.std(msv) > 0.01   # V is not normalised


def test_varlen_recipe():
    w = W.make_workload("varlen")
    lengths, cu = w["lengths"], w["cu_seqlens"]
    assert len(lengths) == 64 and lengths.min() >= 256 and lengths.max() <= 1025
    assert cu.dtype == np.int32 and cu[0] == 0
    np.testing.assert_array_equal(np.diff(cu), lengths)
    assert w["q"].shape == (int(cu[-1]), 25, 128)
    assert w["max_seqlen"] == lengths.max()
    np.testing.assert_array_equal(lengths, W.varlen_lengths(64, 256, 1025, 4))


def test_flop_formulas():
    assert W.WORKLOADS["prefill8k"].flops() == pytest.approx(2 * 8192**2 * 128 * 32)
    assert W.WORKLOADS["vit"].flops() == pytest.approx(4 * 1025**2 * 128 * 25 * 32)
    assert W.varlen_flops([2, 3], 4, 8, False) == 4 * 8 * 4 * 13


def test_band_pair_count():
    # Closed forms, then brute force over a grid of small shapes.
    assert W.band_pairs(50, 50, (None, 0)) == 50 * 51 // 2
    assert W.band_pairs(30, 70, (None, None)) == 30 * 70
    assert W.band_pairs(40, 40, (0, 0)) == 40
    N, w = 8192, 2048
    assert W.band_pairs(N, N, (w - 1, 0)) == (w - 1) * w // 2 + (N - w + 1) * w
    assert W.WORKLOADS["band8k"].flops() == pytest.approx(4.0 * 14681088 * 128 * 32)
    for Nq in (1, 5, 9):
        for Nk in (1, 4, 11):
            for window in [(None, 0), (2, 3), (0, None), (7, 0), (0, 0), (20, 20)]:
                left, right = window
                n = 0
                for i in range(Nq):
                    for j in range(Nk):
                        p = i + Nk - Nq
                        n += (left is None or j >= p - left) and (right is None or j <= p + right)
                assert W.band_pairs(Nq, Nk, window) == n, (Nq, Nk, window)


def test_f16_rne_hand_picked():
    x = np.array([1.0, 65504.0, 1 / 3, 2.0**-24, 1 + 2.0**-11, 1 + 3 * 2.0**-11, -2.5, 0.0],
                 dtype=np.float32)
    want = [0x3C00, 0x7BFF, 0x3555, 0x0001, 0x3C00, 0x3C02, 0xC100, 0x0000]
    assert W.f32_to_f16_bits(x).tolist() == want
    assert np.array_equal(W.f16_bits_to_f32(np.array(want, dtype=np.uint16))[[0, 1, 6]],
                          np.array([1.0, 65504.0, -2.5], dtype=np.float32))


def test_f16_matches_torch_conversion():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(7).standard_normal(10000).astype(np.float32) * 50
    ours = W.f32_to_f16_bits(x)
    theirs = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


def test_dense_f16_takes_the_same_draws():
    qb, kb, vb = W.make_dense(1, 9, 2, 32, seed=5)
    qh, kh, vh = W.make_dense(1, 9, 2, 32, seed=5, dtype="f16")
    # both round the same float32 draws: they agree to bf16 precision
    assert np.allclose(W.bf16_bits_to_f32(qb), W.f16_bits_to_f32(qh), rtol=2**-7, atol=1e-6)
    assert not np.array_equal(qb, qh)


def test_padded_workload_recipe():
    wl = W.make_workload("vitpad")
    spec = wl["spec"]
    n = spec.pad_lengths()
    assert wl["mask"].shape == (32, 1025) and n.min() >= 256 and n.max() <= 1025
    assert np.array_equal(wl["mask"].sum(axis=1), n)
    assert np.all(wl["mask"][np.arange(32), n - 1] == 1)
    assert spec.flops() == pytest.approx(4.0 * float(np.sum(n.astype(float) ** 2)) * 128 * 25)


def test_decode_workload_recipe():
    wl = W.make_workload("decode8k")
    spec = wl["spec"]
    assert wl["q"].shape == (16, 1, 32, 128) and wl["k"].shape == (16, 8192, 32, 128)
    assert spec.bytes_compulsory() == 2 * 16 * 8192 * 32 * 128 * 2 + 2 * 16 * 32 * 128 * 2 + 16 * 32 * 4
    rng = np.random.default_rng(spec.seed)
    q = W.f32_to_bf16_bits(rng.standard_normal((16, 1, 32, 128), dtype=np.float32))
    assert np.array_equal(q, wl["q"])


def test_local_pair_count_matches_the_oracle_mask():
    from oracle import local_pairs
    for args in [(1608, 8, 40, 2, 2, False), (777, 3, 17, 3, 1, True), (300, 300, 5, 0, 0, True),
                 (50, 0, 7, 1, 2, False), (129, 70, 13, 0, 0, True)]:
        assert W.local_pairs_count(*args) == local_pairs(*args), args
