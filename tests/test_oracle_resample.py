"""Pins of the oracle's normalise / ESS / systematic-resampling / remap steps (CPU only).

Against: hand-worked fixtures (tests/golden/), closed forms, library routines the oracle does
not use (numpy.searchsorted, scipy logsumexp/softmax, numpy.bincount), exact integration over
the uniform, and structural invariants of evict-and-duplicate.
"""
import math

import numpy as np
import pytest
import scipy.special

import oracle
from golden_io import load


def _resample(lw, u, mode="always", ess_frac=0.5, prev=None):
    lw = np.asarray(lw, np.float64)
    N = lw.size
    prev = np.full(N, -math.log(N)) if prev is None else np.asarray(prev, np.float64)
    return oracle.resample_request(lw, prev, u, mode, ess_frac)


# ---------------------------------------------------------------- golden hand cases
def test_systematic_hand_cases():
    for case in load("systematic_hand.txt"):
        w = np.array(case["w"])
        with np.errstate(divide="ignore"):
            lw = np.log(w)
        lw[np.isneginf(lw)] = -1e4                      # exp underflows to exactly 0
        out = _resample(lw, case["u"][0])
        assert out["resampled"] == 1
        assert out["ancestors"].tolist() == [int(a) for a in case["ancestors"]], case
        assert out["ess"] == pytest.approx(case["ess"][0], rel=1e-15)


def test_best_particle_copied_to_all():
    case = load("best_particle_copied.txt")[0]
    out = _resample(case["log_w"], case["u"][0])
    assert out["ancestors"].tolist() == [int(a) for a in case["ancestors"]]
    assert out["ess"] == pytest.approx(case["ess"][0], rel=1e-15)


# ---------------------------------------------------------------- normalise / ESS
def test_uniform_weights_identity_and_ess():
    for N in (1, 2, 8, 32, 256):
        for u in (0.0, 0.3, 1.0 - 2.0 ** -24):
            out = _resample(np.zeros(N), u)
            assert out["ancestors"].tolist() == list(range(N))
            assert out["ess"] == N
            assert out["log_norm"] == 0.0
            assert np.all(out["log_weights"] == -math.log(N))


def test_normaliser_and_ess_closed_forms():
    rng = np.random.default_rng(11)
    for N in (3, 16, 100):
        lw = rng.normal(0, 2, N)
        prev = rng.normal(0, 1, N)
        prev = prev - scipy.special.logsumexp(prev)     # normalised carried weights
        out = _resample(lw, 0.5, mode="never", prev=prev)
        l = prev + lw
        assert out["log_norm"] == pytest.approx(scipy.special.logsumexp(l), rel=1e-13, abs=1e-13)
        w = np.exp(l - l.max())
        assert out["ess"] == pytest.approx(w.sum() ** 2 / (w ** 2).sum(), rel=1e-12)
        # not resampled: identity, carried weights normalised to LSE = 0
        assert out["ancestors"].tolist() == list(range(N))
        assert scipy.special.logsumexp(out["log_weights"]) == pytest.approx(0.0, abs=1e-12)
        assert np.allclose(out["log_weights"], l - scipy.special.logsumexp(l), atol=1e-12)


def test_dominant_particle_ess_near_one():
    lw = np.zeros(16)
    lw[5] = 100.0
    out = _resample(lw, 0.77)
    assert out["ess"] == pytest.approx(1.0, abs=1e-12)
    assert np.all(out["ancestors"] == 5)


def test_ess_threshold_mode():
    N = 8
    # two particles share all the weight equally: ESS = 2 exactly
    lw = np.full(N, -1e4)
    lw[[2, 6]] = 0.0
    below = _resample(lw, 0.1, mode="ess", ess_frac=0.5)       # 2 < 4: resample
    assert below["resampled"] == 1 and below["ess"] == pytest.approx(2.0, rel=1e-14)
    assert sorted(set(below["ancestors"].tolist())) == [2, 6]
    assert np.all(below["log_weights"] == -math.log(N))
    above = _resample(lw, 0.1, mode="ess", ess_frac=0.25)      # 2 < 2 is false: keep
    assert above["resampled"] == 0
    assert above["ancestors"].tolist() == list(range(N))
    never = _resample(lw, 0.1, mode="never")
    assert never["resampled"] == 0


# ---------------------------------------------------------------- systematic resampling
def _check_systematic(lw, u, out):
    N = lw.size
    W = scipy.special.softmax(lw)
    C = np.cumsum(W)
    U = (np.arange(N) + u) / N
    ref = np.minimum(np.searchsorted(C, U, side="right"), N - 1)
    gap = out["anc_gap"]
    safe = gap > 1e-12
    assert np.array_equal(out["ancestors"][safe], ref[safe])
    anc = out["ancestors"]
    assert np.all(np.diff(anc) >= 0)                            # non-decreasing
    o = np.bincount(anc, minlength=N)
    assert o.sum() == N
    lo = np.floor(N * W - 1e-9)
    hi = np.ceil(N * W + 1e-9)
    assert np.all(o >= lo) and np.all(o <= hi)                  # o_i in {floor, ceil}(N W_i)


def test_systematic_matches_searchsorted_and_offspring_bounds():
    rng = np.random.default_rng(12)
    for N in (1, 2, 5, 32, 257):
        for _ in range(20):
            lw = rng.normal(0, 3, N)
            u = float(np.float32(rng.random()))
            _check_systematic(lw, u, _resample(lw, u))


def test_systematic_is_unbiased_exact_integration():
    # E_u[o_i] = N W_i: integrate the piecewise-constant offspring counts over u in [0,1)
    rng = np.random.default_rng(13)
    for N in (3, 7, 16):
        lw = rng.normal(0, 1.5, N)
        W = scipy.special.softmax(lw)
        C = np.cumsum(W)
        j = np.arange(N)[:, None]
        brk = (N * C[None, :] - j).ravel()
        brk = np.unique(np.concatenate([[0.0, 1.0], brk[(brk > 0) & (brk < 1)]]))
        mean_o = np.zeros(N)
        for a, b in zip(brk[:-1], brk[1:]):
            if b - a < 1e-15:
                continue
            out = _resample(lw, 0.5 * (a + b))
            mean_o += (b - a) * np.bincount(out["ancestors"], minlength=N)
        assert np.allclose(mean_o, N * W, atol=1e-9), (mean_o, N * W)


# ---------------------------------------------------------------- page-table remap
def _rand_table(rng, N, P, num_pages):
    pt = rng.integers(0, num_pages, (N, P)).astype(np.int32)
    pt[rng.random((N, P)) < 0.2] = -1
    pt[:, : P // 2] = pt[0, : P // 2]                           # shared prompt pages
    rc = np.bincount(pt[pt >= 0], minlength=num_pages).astype(np.int32)
    return pt, rc


def test_remap_hand_case():
    c = load("remap_hand.txt")[0]
    pt = np.array([c["row0"], c["row1"], c["row2"]], np.int32)
    out, rc, st = oracle.remap_request(np.array(c["ancestors"], np.int32), pt,
                                       np.array(c["refcount_in"], np.int32))
    assert st == 0
    assert out.tolist() == [list(map(int, c[k])) for k in ("out_row0", "out_row1", "out_row2")]
    assert rc.tolist() == list(map(int, c["refcount_out"]))


def test_remap_bruteforce_recount():
    rng = np.random.default_rng(14)
    for N, P, npg in [(1, 4, 10), (4, 8, 40), (16, 32, 300), (32, 5, 1000)]:
        for _ in range(10):
            pt, rc = _rand_table(rng, N, P, npg)
            anc = np.sort(rng.integers(0, N, N)).astype(np.int32)
            out, rc2, st = oracle.remap_request(anc, pt, rc)
            assert st == 0
            assert np.array_equal(out, pt[anc])                 # numpy fancy indexing
            old = np.bincount(pt[pt >= 0], minlength=npg)
            new = np.bincount(out[out >= 0], minlength=npg)
            assert np.array_equal(rc2, rc + new - old)
            assert rc2.sum() == (out >= 0).sum()                # references conserved


def test_remap_identity_and_all_to_zero():
    rng = np.random.default_rng(15)
    N, P, npg = 8, 12, 200
    pt, rc = _rand_table(rng, N, P, npg)
    out, rc2, st = oracle.remap_request(np.arange(N, dtype=np.int32), pt, rc)
    assert st == 0 and np.array_equal(out, pt) and np.array_equal(rc2, rc)
    out, rc3, st = oracle.remap_request(np.zeros(N, np.int32), pt, rc)
    assert st == 0 and np.all(out == pt[0])
    # closed form: every page ends with N times its count in row 0
    row0 = np.bincount(pt[0][pt[0] >= 0], minlength=npg)
    assert np.array_equal(rc3, rc - np.bincount(pt[pt >= 0], minlength=npg) + N * row0)


def test_remap_rejects_out_of_range():
    pt = np.array([[0, 1], [2, 99]], np.int32)
    rc = np.zeros(10, np.int32)
    rc[[0, 1, 2]] = 1
    assert oracle.remap_request(np.array([0, 1], np.int32), pt, rc)[2] == -1     # page 99
    assert oracle.remap_request(np.array([0, 5], np.int32), pt[:, :1], rc)[2] == -1  # anc 5
