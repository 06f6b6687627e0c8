"""Pins of the oracle's optional potential (CPU only).

The SMC-SD page ("Faster LLM Inference via Sequential Monte Carlo", section 5) names
constrained generation and reward-weighted decoding as distributions the same resampling
machinery can target. Reading: the target becomes p times a potential phi >= 0, so each
particle's incremental log weight gains log phi (given per particle and round; -inf removes a
particle). These checks tie the oracle to that reading through quantities other than its own
formula: the per-sequence weight p*phi/q on the V = 4, K = 2 toy model, the exact resampled
law converging to the tilted target p*phi/Z instead of p, invariance of the normalised weights
under a constant potential, and a removed particle never being an ancestor.
"""
import itertools
import math

import numpy as np
import pytest

import oracle
from test_oracle_law import V, _round_inputs, _toy, _tv


def _phi(seed=8):
    rng = np.random.default_rng(seed)
    return rng.uniform(0.05, 2.0, V * V)          # phi(s) > 0 on the 16 sequences


def _with_potential(inp, seqs, log_phi):
    inp = dict(inp)
    inp["log_potential"] = log_phi[seqs].astype(np.float32)
    return inp


def test_weight_is_target_times_potential_over_draft():
    tables, p, q = _toy()
    phi = _phi()
    seqs = np.arange(V * V)[None, :]
    lphi = np.log(phi).astype(np.float32)
    out = oracle.round(_with_potential(_round_inputs(tables, seqs), seqs, lphi), mode="never")
    w = np.exp(out["log_w_incr"][0])
    # phi enters as the float32 log potential, so compare against exactly that value
    assert np.allclose(w, p / q * np.exp(lphi.astype(np.float64)), rtol=1e-12)


def test_exact_law_converges_to_tilted_target():
    tables, p, q = _toy()
    phi = _phi()
    lphi = np.log(phi).astype(np.float32)
    tilted = p * np.exp(lphi.astype(np.float64))
    tilted /= tilted.sum()
    tvs, tvs_p = [], []
    for N in range(1, 5):
        seqs = np.array(list(itertools.product(range(V * V), repeat=N)))
        out = oracle.round(_with_potential(_round_inputs(tables, seqs), seqs, lphi), mode="never")
        W = np.exp(out["log_weights"])
        prob = np.prod(q[seqs], axis=1)
        L = np.zeros(V * V)
        for i in range(N):
            np.add.at(L, seqs[:, i], prob * W[:, i])
        assert L.sum() == pytest.approx(1.0, abs=1e-12)
        if N == 1:
            assert np.allclose(L, q, atol=1e-14)
        tvs.append(_tv(L, tilted))
        tvs_p.append(_tv(L, p))
    assert all(a > b for a, b in zip(tvs, tvs[1:])), tvs
    assert tvs[-1] < 0.5 * tvs[0]
    # the population moves toward p*phi/Z, not toward p
    assert tvs[-1] < tvs_p[-1]


def test_constant_potential_leaves_normalised_weights():
    tables, p, q = _toy()
    rng = np.random.default_rng(3)
    seqs = rng.integers(0, V * V, size=(3, 7))
    base = oracle.round(_round_inputs(tables, seqs), mode="never")
    c = np.float32(-2.75)
    inp = _round_inputs(tables, seqs)
    inp["log_potential"] = np.full(seqs.shape, c, np.float32)
    out = oracle.round(inp, mode="never")
    assert np.allclose(out["log_w_incr"], base["log_w_incr"] + float(c), atol=1e-12)
    assert np.allclose(out["log_norm"], base["log_norm"] + float(c), atol=1e-12)
    assert np.allclose(out["log_weights"], base["log_weights"], atol=1e-12)
    assert np.allclose(out["ess"], base["ess"], rtol=1e-12)


def test_removed_particle_is_never_an_ancestor():
    tables, p, q = _toy()
    rng = np.random.default_rng(4)
    N = 9
    seqs = rng.integers(0, V * V, size=(64, N))
    inp = _round_inputs(tables, seqs)
    lpot = np.zeros(seqs.shape, np.float32)
    dead = rng.integers(0, N, size=64)
    lpot[np.arange(64), dead] = -np.inf
    inp["log_potential"] = lpot
    inp["uniform"] = rng.uniform(0, 1, 64).astype(np.float32)
    out = oracle.round(inp, mode="always")
    anc = out["ancestors"]
    assert not np.any(anc == dead[:, None])
    assert np.all(np.isneginf(out["log_w_incr"][np.arange(64), dead]))
    # the other particles keep their usual weights
    base = oracle.round(_round_inputs(tables, seqs), mode="never")
    keep = np.ones(seqs.shape, bool)
    keep[np.arange(64), dead] = False
    assert np.array_equal(out["log_w_incr"][keep], base["log_w_incr"][keep])
