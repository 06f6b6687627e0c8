"""Pins of the oracle's standard speculative-decoding verification (CPU only).

The SMC-SD page ("Faster LLM Inference via Sequential Monte Carlo", section 1) describes the
baseline it replaces: a draft proposes tokens, the target verifies them, and the first
rejection discards the rest of the block. The oracle reads this as standard speculative
sampling (accept with min(1, p/q), resample the first rejected position from
max(p - q, 0), bonus draw from p when everything is accepted). The checks below do not retype
that rule: they compare the acceptance threshold and the residual law with torch.softmax in
float64, and test the defining property of speculative sampling -- the first emitted token
is distributed exactly as p -- by a chi-square test over 200 000 sequences, plus p = q
(everything accepted) and hand-worked residual cases.
"""
import math

import numpy as np
import pytest
import torch
from scipy import stats

import oracle


def _softmax(z, T=1.0):
    return torch.softmax(torch.from_numpy(np.asarray(z, np.float64)) / T, -1).numpy()


def _inputs(zp, zq, tokens, T, acc_u, res_u, gumbel=None):
    """zp [M, K+1, V], zq [M, K, V] float32 as M particles of one request each."""
    M, K1, V = zp.shape
    K = K1 - 1
    return dict(target=zp.reshape(M, 1, K1, V).astype(np.float32),
                draft=zq.reshape(M, 1, K, V).astype(np.float32),
                tokens=tokens.reshape(M, 1, K).astype(np.int32),
                temperature=np.full(M, T, np.float32),
                gumbel=(np.zeros((M, 1, V), np.float32) if gumbel is None
                        else gumbel.reshape(M, 1, V).astype(np.float32)),
                accept_uniform=acc_u.reshape(M, 1, K).astype(np.float32),
                residual_uniform=res_u.reshape(M, 1).astype(np.float32))


def test_identical_distributions_accept_everything():
    rng = np.random.default_rng(0)
    M, K, V = 50, 4, 37
    z = rng.normal(0, 2, (M, K + 1, V)).astype(np.float32)
    g = rng.gumbel(size=(M, V)).astype(np.float32)
    tok = rng.integers(0, V, (M, K))
    out = oracle.sd_verify(_inputs(z, z[:, :K].copy(), tok, 0.8,
                                   rng.uniform(0, 1, (M, K)) * 0.999999, rng.uniform(0, 1, M), g))
    assert np.all(out["n_accepted"] == K)
    bonus = np.argmax(z[:, K].astype(np.float64) / np.float32(0.8) + g, axis=-1)
    assert np.array_equal(out["next_token"][:, 0], bonus)


def test_acceptance_threshold_is_min_one_ratio():
    rng = np.random.default_rng(1)
    V = 9
    for trial in range(40):
        zp = rng.normal(0, 1.5, (1, 2, V)).astype(np.float32)
        zq = rng.normal(0, 1.5, (1, 1, V)).astype(np.float32)
        x = int(rng.integers(0, V))
        T = float(rng.choice([0.6, 1.0, 1.3]))
        T32 = float(np.float32(T))
        p = _softmax(zp[0, 0], T32)
        q = _softmax(zq[0, 0], T32)
        m = min(1.0, p[x] / q[x])
        tok = np.array([[x]])
        below = oracle.sd_verify(_inputs(zp, zq, tok, T, np.array([m * (1 - 1e-6)]), np.array([0.5])))
        assert below["n_accepted"][0, 0] == 1
        if m < 1 - 1e-6:
            above = oracle.sd_verify(_inputs(zp, zq, tok, T, np.array([m * (1 + 1e-6)]), np.array([0.5])))
            assert above["n_accepted"][0, 0] == 0


def test_residual_law_matches_positive_part_of_p_minus_q():
    rng = np.random.default_rng(2)
    V = 12
    zp = rng.normal(0, 1.2, (1, 2, V)).astype(np.float32)
    zq = rng.normal(0, 1.2, (1, 1, V)).astype(np.float32)
    p, q = _softmax(zp[0, 0]), _softmax(zq[0, 0])
    x = int(np.argmin(p / q))                       # a token with p/q < 1
    assert p[x] / q[x] < 0.99
    r = np.maximum(p - q, 0.0)
    r /= r.sum()
    G = 20000
    b = (np.arange(G) + 0.5) / G
    M = G
    inp = _inputs(np.repeat(zp, M, 0), np.repeat(zq, M, 0), np.full((M, 1), x), 1.0,
                  np.full(M, 0.999999), b)
    out = oracle.sd_verify(inp)
    assert np.all(out["n_accepted"] == 0)
    hist = np.bincount(out["next_token"][:, 0], minlength=V) / G
    assert np.abs(hist - r).max() <= 1.0 / G + 1e-12
    assert np.all(hist[r == 0] == 0)


def test_hand_worked_residuals():
    # p = (0.6, 0.4, ~0), q = (0.1, 0.1, 0.8): residual (0.5, 0.3, 0) / 0.8
    zp = np.log(np.array([[[0.6, 0.4, 1e-30], [1.0, 1.0, 1.0]]]))
    zq = np.log(np.array([[[0.1, 0.1, 0.8]]]))
    tok = np.array([[2]])                            # p/q ~ 0: always rejected
    for b, want in ((0.0, 0), (0.62, 0), (0.63, 1), (0.999, 1)):
        out = oracle.sd_verify(_inputs(zp, zq, tok, 1.0, np.array([0.5]), np.array([b])))
        assert out["n_accepted"][0, 0] == 0 and out["next_token"][0, 0] == want, (b, out)
    # the chosen token's cumulative-sum interval and its neighbours
    out = oracle.sd_verify(_inputs(zp, zq, tok, 1.0, np.array([0.5]), np.array([0.3])))
    assert out["next_token"][0, 0] == 0
    assert out["res_lo"][0, 0] == pytest.approx(0.3, abs=1e-6)        # b is float32
    assert out["res_hi"][0, 0] == pytest.approx((0.5 - 0.24) / 0.8, abs=1e-6)
    assert (out["res_below"][0, 0], out["res_above"][0, 0]) == (-1, 1)
    out = oracle.sd_verify(_inputs(zp, zq, tok, 1.0, np.array([0.5]), np.array([0.9])))
    assert out["next_token"][0, 0] == 1
    assert out["res_lo"][0, 0] == pytest.approx((0.72 - 0.5) / 0.8, abs=1e-6)
    assert out["res_hi"][0, 0] == pytest.approx(0.1, abs=1e-6)
    assert (out["res_below"][0, 0], out["res_above"][0, 0]) == (0, -1)
    # a boundary: b * R exactly on C_0 = 0.5 (R = 0.8, b = 0.625) goes to the next token
    out = oracle.sd_verify(_inputs(zp, zq, tok, 1.0, np.array([0.5]), np.array([0.625])))
    assert out["res_gap"][0, 0] < 1e-6


@pytest.mark.parametrize("K", [1, 3])
def test_first_emitted_token_follows_target(K):
    """Speculative sampling is exact: the first emitted token is a draw from p_0."""
    rng = np.random.default_rng(10 + K)
    V, M = 8, 200000
    zp0 = rng.normal(0, 1.5, V)
    zq0 = zp0 + rng.normal(0, 1.0, V)
    p0, q0 = _softmax(zp0), _softmax(zq0)
    zp = np.broadcast_to(rng.normal(0, 1.5, (K + 1, V)), (M, K + 1, V)).copy()
    zq = np.broadcast_to(rng.normal(0, 1.5, (K, V)), (M, K, V)).copy()
    zp[:, 0] = zp0
    zq[:, 0] = zq0
    zp, zq = zp.astype(np.float32), zq.astype(np.float32)
    p0, q0 = _softmax(zp[0, 0]), _softmax(zq[0, 0])
    tok = rng.integers(0, V, (M, K))
    tok[:, 0] = rng.choice(V, size=M, p=q0)          # x_0 ~ q_0
    out = oracle.sd_verify(_inputs(zp, zq, tok, 1.0, rng.uniform(0, 1, (M, K)),
                                   rng.uniform(0, 1, M), rng.gumbel(size=(M, V))))
    first = np.where(out["n_accepted"][:, 0] >= 1, tok[:, 0], out["next_token"][:, 0])
    counts = np.bincount(first, minlength=V)
    chi2, pval = stats.chisquare(counts, M * p0)
    assert pval > 1e-3, (chi2, pval)
    # and not the draft's law
    _, pval_q = stats.chisquare(counts, M * q0)
    assert pval_q < 1e-6
