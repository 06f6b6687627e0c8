"""Pins of the oracle's per-row arithmetic against closed forms, invariants and library
routines the oracle does not use (CPU only).

Each test names what a plausible mistake would break:
  * log-softmax normaliser: temperature applied wrongly, no max shift (overflow), wrong log;
  * TV: missing 1/2, wrong normalisation, sign;
  * Gumbel-max bonus: wrong noise sign or row, tie order, not a draw from p.
"""
import math

import numpy as np
import pytest
import scipy.stats
import torch

import oracle


def bf16_bits(x) -> np.ndarray:
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- log-softmax normaliser
@pytest.mark.parametrize("V", [1, 7, 1000, 32000])
@pytest.mark.parametrize("T", [0.5, 0.7, 1.0])
def test_lse_constant_row_closed_form(V, T):
    # constant row c: LSE(c/T) = c/T + log V; c = 500 at T = 0.5 overflows exp without a shift
    for c in (0.0, -3.25, 500.0):
        z = np.full(V, c, np.float32)
        got = oracle.row_logsumexp(z, T)
        want = c / T + math.log(V)
        assert got == pytest.approx(want, rel=1e-13, abs=1e-12)


def test_lse_shift_invariance():
    rng = np.random.default_rng(1)
    # values on a 1/256 grid so that z + 1024 is exact in binary32
    z = (np.round(rng.normal(0, 3, 5000) * 256) / 256).astype(np.float32)
    for T in (0.6, 1.0, 1.3):
        a = oracle.row_logsumexp(z, T)
        b = oracle.row_logsumexp(z + np.float32(1024.0), T)
        assert b - a == pytest.approx(1024.0 / T, rel=1e-12)


def test_lse_two_point_and_single():
    for a, b, T in [(0.0, 0.0, 1.0), (3.5, -2.0, 1.0), (-7.0, 4.0, 0.7), (90.0, 89.5, 0.5)]:
        z = np.array([a, b], np.float32)
        x, y = a / T, b / T
        want = max(x, y) + math.log1p(math.exp(-abs(x - y)))
        assert oracle.row_logsumexp(z, T) == pytest.approx(want, rel=1e-14, abs=1e-14)
    # V = 1: the only token has log-probability 0, i.e. LSE = z/T
    assert oracle.row_logsumexp(np.array([2.5], np.float32), 0.8) == pytest.approx(2.5 / 0.8)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_lse_matches_torch_float64(dtype):
    rng = np.random.default_rng(2)
    for V, T in [(11, 1.0), (4097, 0.7), (32000, 1.2)]:
        x = rng.normal(0, 3, V).astype(np.float32)
        if dtype == "bf16":
            z = bf16_bits(x)
            vals = bf16_values(z)
        else:
            z = x
            vals = x.astype(np.float64)
        want = torch.logsumexp(torch.from_numpy(vals) / T, dim=0).item()
        assert oracle.row_logsumexp(z, T) == pytest.approx(want, rel=1e-13, abs=1e-13)


# ---------------------------------------------------------------- total variation
def test_tv_identical_rows_is_zero():
    rng = np.random.default_rng(3)
    z = rng.normal(0, 3, 777).astype(np.float32)
    assert oracle.row_tv(z, z, 1.0) == 0.0
    zb = bf16_bits(z)
    assert oracle.row_tv(zb, zb, 0.6) == 0.0


def test_tv_two_point_closed_form():
    for (a0, a1), (b0, b1), T in [((0, 1), (1, 0), 1.0), ((2, -1), (0.5, 0.25), 0.7),
                                  ((0, 0), (0, 3), 1.2)]:
        zp = np.array([a0, a1], np.float32)
        zq = np.array([b0, b1], np.float32)
        p1 = 1.0 / (1.0 + math.exp(-(a1 - a0) / T))
        q1 = 1.0 / (1.0 + math.exp(-(b1 - b0) / T))
        assert oracle.row_tv(zp, zq, T) == pytest.approx(abs(p1 - q1), rel=1e-13, abs=1e-15)


def test_tv_disjoint_support_is_one():
    V = 100
    zp = np.zeros(V, np.float32)
    zq = np.zeros(V, np.float32)
    zp[0] = 60.0
    zq[1] = 60.0
    # p and q each put all but ~V e^-60 of their mass on different tokens
    assert oracle.row_tv(zp, zq, 1.0) == pytest.approx(1.0, abs=1e-12)


def test_tv_three_formulas_agree_with_torch_softmax():
    rng = np.random.default_rng(4)
    for V, T, s in [(50, 1.0, 0.3), (5000, 0.7, 1.5), (20000, 1.2, 0.05)]:
        zp = rng.normal(0, 3, V).astype(np.float32)
        zq = (zp + rng.normal(0, s, V)).astype(np.float32)
        p = torch.softmax(torch.from_numpy(zp.astype(np.float64)) / T, 0)
        q = torch.softmax(torch.from_numpy(zq.astype(np.float64)) / T, 0)
        half_l1 = 0.5 * (p - q).abs().sum().item()
        pos_part = torch.clamp(p - q, min=0).sum().item()
        one_minus_min = 1.0 - torch.minimum(p, q).sum().item()
        got = oracle.row_tv(zp, zq, T)
        for want in (half_l1, pos_part, one_minus_min):
            assert got == pytest.approx(want, rel=1e-10, abs=1e-13)
        assert 0.0 <= got <= 1.0


def test_tv_temperature_is_applied_to_both_rows():
    rng = np.random.default_rng(5)
    zp = (np.round(rng.normal(0, 3, 300) * 64) / 64).astype(np.float32)
    zq = (np.round(rng.normal(0, 3, 300) * 64) / 64).astype(np.float32)
    # T = 2 on z equals T = 1 on z/2 (exact halving in binary32)
    a = oracle.row_tv(zp, zq, 2.0)
    b = oracle.row_tv(zp / np.float32(2), zq / np.float32(2), 1.0)
    assert a == pytest.approx(b, rel=1e-14)
    assert abs(a - oracle.row_tv(zp, zq, 1.0)) > 1e-3


# ---------------------------------------------------------------- Gumbel-max bonus token
def test_gumbel_zero_noise_is_plain_argmax_first_index():
    rng = np.random.default_rng(6)
    for V in (1, 2, 9, 1000):
        z = rng.integers(-3, 4, V).astype(np.float32)       # many ties at the max
        g = np.zeros(V, np.float32)
        idx, gap = oracle.row_gumbel_argmax(z, g, 0.9)
        assert idx == int(np.argmax(z))                     # numpy: first maximal index
        if V > 1 and np.sum(z == z.max()) > 1:
            assert gap == 0.0


def test_gumbel_key_ties_go_to_lowest_index():
    z = np.array([1.0, 3.0, 2.0, 3.0], np.float32)
    g = np.array([0.0, -1.0, 0.0, -1.0], np.float32)
    assert oracle.row_gumbel_argmax(z, g, 1.0)[0] == 1
    g2 = np.array([2.0, 0.0, 0.0, 0.0], np.float32)         # 1+2 == 3+0: tie between 0, 1, 3
    assert oracle.row_gumbel_argmax(z, g2, 1.0)[0] == 0


def test_gumbel_noise_sign_and_temperature():
    z = np.array([0.0, 1.0], np.float32)
    # key = z/T + g: a noise of +2 on token 0 beats z=1 at T=1 but not at T=0.25 (1/T=4)
    g = np.array([2.0, 0.0], np.float32)
    assert oracle.row_gumbel_argmax(z, g, 1.0)[0] == 0
    assert oracle.row_gumbel_argmax(z, g, 0.25)[0] == 1


def test_gumbel_keys_are_exact_not_binary32():
    # key = z/T + G as a real number. z = 1 at T = 3 gives 1/3; token 1 has no logit and noise
    # fl32(1/3) = 1/3 + 9.93e-9. Exactly, token 1 is larger by 9.93e-9; a binary32 key
    # fma(z, fl32(1/T), G) would make the two equal (and pick token 0 by the tie rule).
    g1 = np.float32(1.0) / np.float32(3.0)
    z = np.array([1.0, 0.0], np.float32)
    g = np.array([0.0, g1], np.float32)
    idx, gap = oracle.row_gumbel_argmax(z, g, 3.0)
    assert idx == 1
    assert gap == pytest.approx(float(g1) - 1.0 / 3.0, rel=1e-6) and 9e-9 < gap < 1.1e-8
    # the gap is the distance to the runner-up, +inf with one token
    assert oracle.row_gumbel_argmax(np.array([4.0, 1.0, 2.5], np.float32),
                                    np.zeros(3, np.float32), 0.5)[1] == pytest.approx(3.0)
    assert oracle.row_gumbel_argmax(np.array([4.0], np.float32), np.zeros(1, np.float32),
                                    1.0)[1] == float("inf")


def test_gumbel_max_draws_follow_target_softmax():
    # The bonus token is a draw from p = softmax(z/T): chi-square over many noise rows.
    rng = np.random.default_rng(7)
    V, T, M = 6, 0.8, 60000
    z = np.array([0.3, -1.0, 1.2, 0.0, 2.0, -0.5], np.float32)
    U = np.clip(rng.random((M, V)), np.finfo(np.float32).tiny, 1 - 2.0 ** -24)
    G = (-np.log(-np.log(U))).astype(np.float32)
    counts = np.zeros(V)
    for m in range(M):
        counts[oracle.row_gumbel_argmax(z, G[m], T)[0]] += 1
    p = torch.softmax(torch.from_numpy(z.astype(np.float64)) / T, 0).numpy()
    stat, pval = scipy.stats.chisquare(counts, M * p)
    assert pval > 1e-3, (counts, M * p)
    # and it is not the draft-free argmax: every token is drawn
    assert np.all(counts > 0)
