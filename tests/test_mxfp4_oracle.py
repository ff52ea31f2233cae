"""Pins of the oracle's MXFP4 decode and of the prepared 4-bit index vectors (CPU).

"Sparse Attention", Chapter 4 (FP4 scorer): 4-bit index vectors with scales. The format is
OCP MXFP4: E2M1 elements, one E8M0 scale per 32 elements.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import msa_case, mxfp4
from synth import msa_inputs as mi


def test_e2m1_values_are_the_formats_published_set():
    # the OCP microscaling format's E2M1 value set: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6
    # for codes 0..7, the same negated for codes 8..15 (code 8 is -0)
    pub = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    got = mxfp4.e2m1_value(np.arange(16))
    assert list(got[:8]) == pub
    assert list(-got[8:]) == pub
    assert np.signbit(got[8])


def test_e8m0_decode_matches_torch():
    codes = np.arange(255, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    np.testing.assert_array_equal(mxfp4.e8m0_value(codes), want)
    assert np.isnan(mxfp4.e8m0_value(np.array([255])))[0]


def test_nibble_order_and_scale_groups():
    packed = np.zeros((1, 32), dtype=np.uint8)
    packed[0, 0] = 0x21          # element 0: code 1 (0.5), element 1: code 2 (1.0)
    packed[0, 16] = 0xF7         # element 32: code 7 (6.0), element 33: code 15 (-6.0)
    scales = np.array([[128, 125]], dtype=np.uint8)   # 2^1 for elements 0..31, 2^-2 after
    v = mxfp4.dequantize(packed, scales)
    assert v.shape == (1, 64)
    assert (v[0, 0], v[0, 1], v[0, 32], v[0, 33]) == (1.0, 2.0, 1.5, -1.5)
    assert np.count_nonzero(v) == 4


def _brute_force(x: np.ndarray) -> np.ndarray:
    """Nearest representable value per element, found by trying every candidate: the group
    exponent X is the one that puts amax / 2^X in [4, 8); then every magnitude of the set is
    tried, the nearest kept, a tie going to the even code, anything past 6 taking 6."""
    pub = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    out = np.empty_like(x)
    for r in range(x.shape[0]):
        for g0 in range(0, x.shape[1], 32):
            grp = x[r, g0:g0 + 32]
            amax = float(np.max(np.abs(grp)))
            xe = 0
            if amax > 0:
                xe = -200
                while amax / 2.0 ** (xe + 1) >= 4.0:
                    xe += 1
            for i, val in enumerate(grp):
                m = abs(float(val)) / 2.0 ** xe
                best = 0
                for c in range(8):
                    d, db = abs(m - pub[c]), abs(m - pub[best])
                    if d < db or (d == db and c % 2 == 0 and best % 2 == 1):
                        best = c
                out[r, g0 + i] = (-1.0 if val < 0 else 1.0) * pub[best] * 2.0 ** xe
    return out


@pytest.mark.parametrize("seed", [0, 1])
def test_prepared_vectors_are_nearest_values(seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((24, 64)).astype(np.float32) * np.exp2(rng.integers(-6, 6, (24, 1)))
    # midpoints and saturation on purpose: exact ties at 2^X * {0.25, 0.75, 1.25, 1.75, 2.5,
    # 3.5, 5}, values between 6 and 8, an all-zero group
    x[:2, :32] = 0.0             # groups whose scale is 2^0 (amax in [4, 8))
    x[0, :8] = np.array([4.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    x[1, :3] = np.array([7.9, -7.0, 6.5], np.float32)
    x[2, 32:] = 0.0
    packed, scales = mi.to_mxfp4(x)
    got = mxfp4.dequantize(packed.numpy(), scales.numpy())
    np.testing.assert_array_equal(got, _brute_force(x.astype(np.float64)))
    assert got[0, 1] == 0.0 and got[0, 2] == 1.0 and got[0, 7] == 4.0   # ties to even
    assert got[1, 0] == 6.0 and got[1, 1] == -6.0                      # saturation
    assert scales.numpy()[2, 1] == 127 and not got[2, 32:].any()


def test_dequantised_dot_products_are_exact():
    """The oracle's fp64 dot product of two MXFP4 rows equals the integer-arithmetic sum over
    codes and exponents (so it is the exact value), and that value is an fp32 number: a
    kernel that sums the products in fp32 without loss must return it bit for bit."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((16, 64)).astype(np.float32)
    packed, scales = mi.to_mxfp4(x)
    p, s = packed.numpy(), scales.numpy()
    v = mxfp4.dequantize(p, s)
    codes = mxfp4.unpack_codes(p).astype(int)
    twice = [0, 1, 2, 3, 4, 6, 8, 12]          # 2 * magnitude of codes 0..7, integers
    for a in range(0, 16, 3):
        for b in range(1, 16, 5):
            exact = Fraction(0)
            for d in range(64):
                ia, ib = codes[a, d], codes[b, d]
                sign = (-1) ** (((ia >> 3) + (ib >> 3)) & 1)
                e = int(s[a, d // 32]) + int(s[b, d // 32]) - 254 - 2
                exact += sign * twice[ia & 7] * twice[ib & 7] * Fraction(2) ** e
            dot = float(v[a] @ v[b])
            assert Fraction(dot) == exact
            assert float(np.float32(dot)) == dot


def test_case_oracle_on_mxfp4_proxies():
    cfg = mi.custom(name="i4", n_q=(300,), n_k=(900,), hq=4, hkv=2, topk=4, dp=64,
                    idx_dtype="mxfp4")
    case = mi.make_case(cfg, seed=0)
    assert case.q_idx.shape == (300, 2, 32) and case.q_idx_scale.shape == (300, 2, 2)
    out = msa_case.run(case, want_output=False)
    pos = np.arange(300) + 600
    assert (out.topk_idx[:, :, 0] == (pos // 128)[:, None]).all()    # local block forced
    # every finite proxy block score is an fp32 number (exact sums, see above)
    sc = out.scores[0]
    fin = sc[np.isfinite(sc)]
    np.testing.assert_array_equal(fin.astype(np.float32).astype(np.float64), fin)


def test_planted_mistakes_fail_a_pin(monkeypatch):
    """Each plausible slip in the decode (nibble order, scale bias, sign, group width) makes
    one of the pins above fail."""
    def pins_hold():
        try:
            test_e2m1_values_are_the_formats_published_set()
            test_e8m0_decode_matches_torch()
            test_nibble_order_and_scale_groups()
            test_prepared_vectors_are_nearest_values(0)
        except AssertionError:
            return False
        return True

    assert pins_hold()
    good_unpack, good_e2m1, good_e8m0 = mxfp4.unpack_codes, mxfp4.e2m1_value, mxfp4.e8m0_value

    def swapped(p):
        c = good_unpack(p)
        return np.stack([c[..., 1::2], c[..., 0::2]], axis=-1).reshape(c.shape)
    monkeypatch.setattr(mxfp4, "unpack_codes", swapped)
    assert not pins_hold()
    monkeypatch.setattr(mxfp4, "unpack_codes", good_unpack)
    monkeypatch.setattr(mxfp4, "e8m0_value", lambda c: good_e8m0(c) * 2.0)
    assert not pins_hold()
    monkeypatch.setattr(mxfp4, "e8m0_value", good_e8m0)
    monkeypatch.setattr(mxfp4, "e2m1_value", lambda c: np.abs(good_e2m1(c)))
    assert not pins_hold()
    monkeypatch.setattr(mxfp4, "e2m1_value", good_e2m1)
    monkeypatch.setattr(mxfp4, "MX_BLOCK", 16)
    with pytest.raises(AssertionError):
        mxfp4.dequantize(np.zeros((1, 32), np.uint8), np.zeros((1, 2), np.uint8))
    monkeypatch.setattr(mxfp4, "MX_BLOCK", 32)
    assert pins_hold()
