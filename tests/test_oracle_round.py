"""Round-level pins of the oracle (CPU only): special cases the pages fix, a hand case,
and the structure of the round's outputs.

  * p == q (draft rows identical to target rows): every importance ratio is 1, so the
    log-weights are exactly 0, ESS = N and systematic resampling is the identity for any u
    (N a power of two) -- "Faster LLM Inference via Sequential Monte Carlo", section 2: each
    particle is weighted by how the target rates its drafted tokens relative to the draft.
  * the bonus position (row K of the target) never enters the weights;
  * out_tokens of new slot j are the K drafted tokens plus the bonus of its ancestor (the
    round yields K+1 tokens per particle, section 2);
  * padding columns beyond V are ignored.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _inputs(R=2, N=8, K=3, V=50, ld=None, seed=0, same=False, dtype="f32"):
    rng = np.random.default_rng(seed)
    ld = V if ld is None else ld
    tgt = np.full((R, N, K + 1, ld), 1e4, np.float32)
    dft = np.full((R, N, K, ld), 1e4, np.float32)
    gum = np.full((R, N, ld), 1e4, np.float32)
    tgt[..., :V] = rng.normal(0, 2, (R, N, K + 1, V))
    dft[..., :V] = tgt[:, :, :K, :V] if same else tgt[:, :, :K, :V] + rng.normal(0, 0.5, (R, N, K, V))
    gum[..., :V] = -np.log(-np.log(rng.uniform(1e-7, 1 - 1e-7, (R, N, V))))
    d = dict(target=tgt, draft=dft, tokens=rng.integers(0, V, (R, N, K)).astype(np.int32),
             temperature=np.array([0.7, 1.3][:R] + [1.0] * max(0, R - 2), np.float32),
             gumbel=gum, uniform=rng.random(R).astype(np.float32),
             log_weights=np.full((R, N), -math.log(N), np.float32))
    if dtype == "bf16":
        for k in ("target", "draft"):
            d[k] = torch.from_numpy(d[k]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    pt = rng.integers(0, 500, (R, N, 6)).astype(np.int32)
    pt[:, :, :3] = pt[:, :1, :3]
    d["page_table"] = pt
    d["refcount"] = np.bincount(pt.ravel(), minlength=600).astype(np.int32)
    return d


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_identical_target_and_draft_gives_uniform_weights(dtype):
    d = _inputs(R=3, N=16, K=4, V=97, same=True, dtype=dtype)
    d["uniform"] = np.array([0.0, 0.5, 1.0 - 2.0 ** -24], np.float32)
    out = oracle.round(d, tv=True)
    assert out["status"] == 0
    assert np.all(out["log_w_incr"] == 0.0)
    assert np.all(out["ess"] == 16.0)
    assert np.all(out["ancestors"] == np.arange(16))
    # carried log-weights are binary32, so logZ = fl32(-log N) + log N (|.| < 1e-7), not 0
    assert np.all(out["log_norm"] == float(np.float32(-math.log(16))) + math.log(16))
    assert np.all(out["tv"] == 0.0)
    assert np.array_equal(out["page_table"], d["page_table"])
    assert np.array_equal(out["refcount"], d["refcount"])


def test_hand_case_v2_k1():
    # p = softmax([a0, a1]/T), q = softmax([b0, b1]/T), token 1: lw = log p1 - log q1
    a0, a1, b0, b1, T = 0.25, 1.5, 1.0, -0.5, 0.8
    d = dict(target=np.array([[[[a0, a1], [3.0, -3.0]]]], np.float32),
             draft=np.array([[[[b0, b1]]]], np.float32),
             tokens=np.array([[[1]]], np.int32), temperature=np.array([T], np.float32),
             gumbel=np.zeros((1, 1, 2), np.float32), uniform=np.array([0.5], np.float32),
             log_weights=np.zeros((1, 1), np.float32))
    out = oracle.round(d, tv=True)
    T = float(np.float32(T))                            # the round sees T as binary32
    lp1 = -math.log1p(math.exp(-(a1 - a0) / T))
    lq1 = -math.log1p(math.exp(-(b1 - b0) / T))
    assert out["log_w_incr"][0, 0] == pytest.approx(lp1 - lq1, rel=1e-13)
    p1, q1 = math.exp(lp1), math.exp(lq1)
    assert out["tv"][0, 0, 0] == pytest.approx(abs(p1 - q1), rel=1e-12)
    assert out["bonus"][0, 0] == 0                      # bonus row [3, -3], zero noise
    assert out["ancestors"][0, 0] == 0 and out["ess"][0] == 1.0


def test_bonus_row_does_not_enter_weights():
    d = _inputs(seed=3)
    a = oracle.round(d)
    d2 = dict(d)
    d2["target"] = d["target"].copy()
    d2["target"][:, :, -1, :] = np.random.default_rng(9).normal(0, 5, d2["target"][:, :, -1, :].shape)
    b = oracle.round(d2)
    assert np.array_equal(a["log_w_incr"], b["log_w_incr"])
    assert not np.array_equal(a["bonus"], b["bonus"])


def test_out_tokens_follow_ancestors():
    d = _inputs(R=4, N=8, K=3, seed=4)
    out = oracle.round(d)
    R, N, K = d["tokens"].shape
    for r in range(R):
        anc = out["ancestors"][r]
        assert np.array_equal(out["out_tokens"][r, :, :K], d["tokens"][r, anc])
        assert np.array_equal(out["out_tokens"][r, :, K], out["bonus"][r, anc])
        assert np.array_equal(out["page_table"][r], d["page_table"][r, anc])


def test_round_matches_row_level_definitions():
    d = _inputs(R=2, N=4, K=2, V=40, seed=5)
    out = oracle.round(d, tv=True)
    for r in range(2):
        T = float(d["temperature"][r])
        for i in range(4):
            s = 0.0
            for k in range(2):
                zp, zq = d["target"][r, i, k], d["draft"][r, i, k]
                x = d["tokens"][r, i, k]
                s += ((float(zp[x]) / T - oracle.row_logsumexp(zp, T))
                      - (float(zq[x]) / T - oracle.row_logsumexp(zq, T)))
                assert out["tv"][r, i, k] == pytest.approx(oracle.row_tv(zp, zq, T), rel=1e-14)
            assert out["log_w_incr"][r, i] == pytest.approx(s, rel=1e-13, abs=1e-13)
            b, _ = oracle.row_gumbel_argmax(d["target"][r, i, 2], d["gumbel"][r, i], T)
            assert out["bonus"][r, i] == b


def test_padding_columns_are_ignored():
    a = oracle.round(_inputs(R=2, N=8, K=3, V=50, ld=None, seed=6), tv=True)
    d = _inputs(R=2, N=8, K=3, V=50, ld=56, seed=6)
    b = oracle.round(d, V=50, tv=True)
    for k in ("log_w_incr", "ancestors", "bonus", "tv", "ess"):
        assert np.array_equal(a[k], b[k]), k


def test_out_of_range_token_is_reported():
    d = _inputs(seed=7)
    d["tokens"][0, 0, 0] = 50
    assert oracle.round(d)["status"] == -1
