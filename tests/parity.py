"""Element-by-element comparison of a GPU round against the CPU oracle on the same inputs.

The bar:
  * bonus tokens: bit-exact everywhere (both sides decide in binary32 on the same key);
  * ancestors: bit-exact wherever the oracle's distance from U_j to the nearest cumulative
    weight C_i is >= 1e-5 (closer than that, fp32 vs fp64 weight arithmetic may legitimately
    pick the neighbour); the request's resample decision must match unless its ESS lies
    within 1e-4*N of the threshold;
  * out_tokens, page tables and refcounts: bit-exact (against the oracle's own remap of the
    GPU's ancestors where a near-tie ancestor was excluded);
  * log_w_incr, log_norm, new log-weights: |d| <= 1e-4 * max(1, |ref|);
  * ESS and TV: |d| <= 1e-4 * |ref| + 1e-6.
"""
from __future__ import annotations

import numpy as np

import oracle

ANC_GAP = 1e-5
REL = 1e-4


def to_numpy(out: dict, requests=None) -> dict:
    res = {}
    for k, v in out.items():
        if v is None or not hasattr(v, "detach"):
            continue
        if k in ("workspace", "error_flags", "refcount"):
            res[k] = v.detach().cpu().numpy()
            continue
        t = v.detach().cpu()
        if requests is not None:
            t = t[list(requests)]
        res[k] = t.numpy()
    return res


def _close(name, got, ref, rel, abs_=0.0, floor=False):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = np.maximum(1.0, np.abs(ref)) if floor else np.abs(ref)
    with np.errstate(invalid="ignore"):
        bad = np.abs(got - ref) > rel * scale + abs_
    # infinities (a particle removed by its potential) must match exactly, NaN nowhere
    bad |= (np.isinf(got) | np.isinf(ref)) & (got != ref)
    bad |= np.isnan(got) | np.isnan(ref)
    if np.any(bad):
        idx = np.argwhere(bad)[:5]
        raise AssertionError("%s: %d mismatches, first %s: got %s ref %s" % (
            name, int(bad.sum()), idx.tolist(), got[tuple(idx.T)], ref[tuple(idx.T)]))


def check_round(host_in: dict, ora: dict, gpu: dict, *, N: int, mode="always",
                ess_frac=0.5, tv=False, pages=True, rc_before=None, rc_after=None) -> dict:
    """Compare one round. ``gpu`` holds numpy copies of the GPU outputs restricted to the same
    requests as ``host_in``. rc_before/rc_after are the full refcount arrays (GPU side)."""
    stats = dict(anc_compared=0, anc_excluded=0)
    _close("log_w_incr", gpu["log_w_incr"], ora["log_w_incr"], REL, floor=True)
    _close("log_norm", gpu["log_norm"], ora["log_norm"], REL, floor=True)
    _close("ess", gpu["ess"], ora["ess"], REL, 1e-6)
    if tv:
        _close("tv", gpu["tv"], ora["tv"], REL, 1e-6)
    bad = np.argwhere(gpu["bonus"] != ora["bonus"])
    if bad.size:
        raise AssertionError("bonus: %d mismatches, first %s (gpu %s, oracle %s, gap %s)" % (
            len(bad), bad[:5].tolist(), gpu["bonus"][tuple(bad[:5].T)],
            ora["bonus"][tuple(bad[:5].T)], ora["bonus_gap"][tuple(bad[:5].T)]))

    R = gpu["ancestors"].shape[0]
    K = host_in["tokens"].shape[2]
    for r in range(R):
        near = mode == "ess" and abs(ora["ess"][r] - ess_frac * N) < 1e-4 * N
        if gpu["resampled"][r] != ora["resampled"][r]:
            if near:
                continue
            raise AssertionError("resampled[%d]: gpu %d oracle %d (ess %g)" % (
                r, gpu["resampled"][r], ora["resampled"][r], ora["ess"][r]))
        safe = ora["anc_gap"][r] >= ANC_GAP
        stats["anc_compared"] += int(safe.sum())
        stats["anc_excluded"] += int((~safe).sum())
        if not np.array_equal(gpu["ancestors"][r][safe], ora["ancestors"][r][safe]):
            j = np.argwhere((gpu["ancestors"][r] != ora["ancestors"][r]) & safe)[:5].ravel()
            raise AssertionError("ancestors[%d] at %s: gpu %s oracle %s gap %s" % (
                r, j.tolist(), gpu["ancestors"][r][j], ora["ancestors"][r][j], ora["anc_gap"][r][j]))
        anc = gpu["ancestors"][r]
        if not (np.all(anc >= 0) and np.all(anc < N) and np.all(np.diff(anc) >= 0)):
            raise AssertionError("ancestors[%d] invalid: %s" % (r, anc))
        if gpu["resampled"][r] == ora["resampled"][r]:
            lw_ref = ora["log_weights"][r]
            _close("log_weights[%d]" % r, gpu["log_weights"][r], lw_ref, REL, floor=True)
        # out_tokens follow the GPU's ancestors exactly
        if "out_tokens" in gpu:
            want = np.concatenate([host_in["tokens"][r][anc], gpu["bonus"][r][anc][:, None]], 1)
            if not np.array_equal(gpu["out_tokens"][r], want):
                raise AssertionError("out_tokens[%d] do not follow the ancestors" % r)
        if pages:
            pt_in = host_in["page_table"][r]
            if np.array_equal(anc, ora["ancestors"][r]):
                pt_ref = ora["page_table"][r]
            else:
                pt_ref, _, _ = oracle.remap_request(anc, pt_in, host_in["refcount"])
            if not np.array_equal(gpu["page_table_out"][r], pt_ref):
                raise AssertionError("page_table_out[%d] mismatch" % r)
    if pages and rc_before is not None and rc_after is not None:
        # exact recount over the pages of the compared requests
        pt_in = host_in["page_table"]
        pt_out = gpu["page_table_out"]
        old = np.bincount(pt_in[pt_in >= 0], minlength=rc_before.size)
        new = np.bincount(pt_out[pt_out >= 0], minlength=rc_before.size)
        touched = (old > 0) | (new > 0)
        want = rc_before.astype(np.int64) + new - old
        if not np.array_equal(rc_after[touched], want[touched]):
            raise AssertionError("refcount mismatch on %d pages" % int((rc_after[touched] != want[touched]).sum()))
        if np.array_equal(gpu["ancestors"], ora["ancestors"]):
            if not np.array_equal(rc_after[touched], ora["refcount"][touched]):
                raise AssertionError("refcount differs from the oracle's")
    return stats
