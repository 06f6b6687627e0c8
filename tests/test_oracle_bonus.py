"""Pins of the oracle's bonus token drawn after resampling (CPU only).

The SMC-SD page (section 2) yields K + 1 tokens per particle and round but leaves open when
the last one is drawn. The in-pass reading draws it per original particle; the alternative
pinned here draws it per new slot j from the target's bonus row (row K) of the slot's
ancestor, with the slot's own noise row, by the Gumbel-max key of the STAND page (method
item 2, k = 1). Pins:
  * identity ancestors reduce it to the in-pass bonus of the round;
  * with the noise rows moved along with the ancestors it reproduces the in-pass bonus of
    the ancestor, slot by slot (row from the ancestor, noise from the slot);
  * law: over many slots sharing one ancestor, the draws follow softmax(row K / T) of that
    ancestor (Gumbel-max), and not any of its other rows;
  * an ancestor outside [0, N) gives -1 and status -1.
"""
import math

import numpy as np
import pytest

import oracle
from test_oracle_round import _inputs


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_identity_ancestors_give_the_in_pass_bonus(dtype):
    d = _inputs(R=2, N=8, K=3, V=50, ld=56, dtype=dtype, seed=3)
    ora = oracle.round(d, V=50, mode="never")
    assert np.array_equal(ora["ancestors"], np.tile(np.arange(8), (2, 1)))
    out = oracle.bonus_resampled(d["target"], d["temperature"], ora["ancestors"], d["gumbel"], V=50)
    assert out["status"] == 0
    assert np.array_equal(out["bonus"], ora["bonus"])


def test_row_follows_the_ancestor_noise_follows_the_slot():
    d = _inputs(R=3, N=8, K=2, V=40, seed=4)
    ora = oracle.round(d, V=40, mode="never")          # in-pass bonus per original particle
    rng = np.random.default_rng(9)
    anc = np.sort(rng.integers(0, 8, (3, 8)), axis=1).astype(np.int32)
    moved = np.take_along_axis(d["gumbel"], anc[:, :, None].astype(np.int64), axis=1)
    out = oracle.bonus_resampled(d["target"], d["temperature"], anc, moved, V=40)
    want = np.take_along_axis(ora["bonus"], anc.astype(np.int64), axis=1)
    assert np.array_equal(out["bonus"], want)
    # with each slot's own (not moved) noise, slots sharing an ancestor draw separately
    own = oracle.bonus_resampled(d["target"], d["temperature"], anc, d["gumbel"], V=40)
    assert not np.array_equal(own["bonus"], want)


def test_law_of_the_draw_is_the_ancestor_bonus_row():
    R, N, K, V = 16, 1024, 2, 5
    T = np.float32(0.8)
    rng = np.random.default_rng(12)
    tgt = np.zeros((R, N, K + 1, V), np.float32)
    tgt[:, :, :K, 0] = 30.0                      # other rows: all mass on token 0
    row = np.array([0.3, -1.0, 1.2, 0.0, -0.4], np.float32)
    tgt[:, 5, K] = row                           # the ancestor's bonus row
    tgt[:, np.arange(N) != 5, K, 4] = 30.0       # other particles' bonus rows: token 4
    anc = np.full((R, N), 5, np.int32)
    g = -np.log(-np.log(rng.uniform(1e-12, 1 - 1e-12, (R, N, V)))).astype(np.float32)
    out = oracle.bonus_resampled(tgt, np.full(R, T, np.float32), anc, g)
    counts = np.bincount(out["bonus"].ravel(), minlength=V)
    p = np.exp(row.astype(np.float64) / float(T))
    p /= p.sum()
    n = R * N
    chi2 = float((((counts - n * p) ** 2) / (n * p)).sum())
    assert chi2 < 20.5, (counts.tolist(), (n * p).round(1).tolist())    # 4 dof, p ~ 4e-4


def test_out_of_range_ancestor():
    d = _inputs(R=1, N=4, K=1, V=10, seed=5)
    anc = np.array([[0, 1, 4, 3]], np.int32)
    out = oracle.bonus_resampled(d["target"], d["temperature"], anc, d["gumbel"], V=10)
    assert out["status"] == -1 and out["bonus"][0, 2] == -1
    assert (out["bonus"][0, [0, 1, 3]] >= 0).all()
