"""Element-by-element comparison of a GPU round against the CPU oracle on the same inputs.

The bar:
  * bonus tokens: bit-exact wherever the oracle's top-2 gap of the key z/T + G (taken in
    double) is >= 1e-5; closer than that, the GPU's binary32 key may order the two the
    other way, so there the GPU's token must only be valid: its exact key lies within 1e-5
    of the oracle's best;
  * ancestors: bit-exact wherever the oracle's distance from U_j to the nearest cumulative
    weight C_i is >= 1e-5 (closer than that, fp32 vs fp64 weight arithmetic may legitimately
    pick the neighbour); the request's resample decision must match unless its ESS lies
    within 1e-4*N of the threshold;
  * out_tokens, page tables and refcounts: bit-exact (against the oracle's own remap of the
    GPU's ancestors where a near-tie ancestor was excluded);
  * log_w_incr, log_norm: |d| <= 1e-4 * |ref| + abs_lw(K); new log-weights (l_i - logZ, two
    such values) |d| <= 1e-4 * |ref| + 2 * abs_lw(K). abs_lw(K) = 2K * 64 * 2^-24 is what a
    relative error alone cannot express near 0: each of the 2K row normalisers is the log of
    a sum of exponentials accumulated in binary32 through at most 64 roundings in a row
    (per-lane sums, the wave tree, the waves, the slices, plus the exp2 and its argument),
    so each is off by at most 64 * 2^-24 in absolute terms;
  * ESS and TV: |d| <= 1e-4 * |ref| + 1e-6.
"""
from __future__ import annotations

import numpy as np

import oracle

ANC_GAP = 1e-5
KEY_GAP = 1e-5
REL = 1e-4


def abs_lw(K: int) -> float:
    """Absolute error bound of a log weight that sums K positions (2K normalisers)."""
    return 2 * K * 64 * 2.0 ** -24


def widen(z: np.ndarray) -> np.ndarray:
    """Logits as float64: float32 as is, bf16 bit patterns (uint16) widened exactly."""
    z = np.asarray(z)
    if z.dtype == np.uint16:
        return (z.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return z.astype(np.float64)


def exact_keys(z_rows, g_rows, T_rows, tokens) -> np.ndarray:
    """z_v/T + G_v in double for the given tokens: z_rows [..., ld] logits, g_rows [..., ld]
    noise, T_rows [...] temperatures, tokens [..., m] -> keys [..., m]."""
    tok = np.asarray(tokens)
    z = np.take_along_axis(widen(z_rows), tok, -1)
    g = np.take_along_axis(np.asarray(g_rows, np.float64), tok, -1)
    return z / np.asarray(T_rows, np.float64)[..., None] + g


def check_bonus(name, got, ref, gap, z_rows, g_rows, T_rows, V) -> dict:
    """Gumbel-max tokens [...]: bit-exact where the oracle's top-2 key gap is >= KEY_GAP, else a
    valid near-tie winner (exact key within KEY_GAP of the oracle's best)."""
    got = np.asarray(got)
    ref = np.asarray(ref)
    if np.any((got < 0) | (got >= V)):
        raise AssertionError("%s: token out of range" % name)
    safe = np.asarray(gap) >= KEY_GAP
    bad = np.argwhere(safe & (got != ref))
    if bad.size:
        raise AssertionError("%s: %d mismatches, first %s (gpu %s, oracle %s, gap %s)" % (
            name, len(bad), bad[:5].tolist(), got[tuple(bad[:5].T)], ref[tuple(bad[:5].T)],
            np.asarray(gap)[tuple(bad[:5].T)]))
    if (~safe).any():
        kg = exact_keys(z_rows, g_rows, T_rows, got[..., None])[..., 0]
        kr = exact_keys(z_rows, g_rows, T_rows, ref[..., None])[..., 0]
        bad = np.argwhere(~safe & (kg < kr - KEY_GAP))
        if bad.size:
            raise AssertionError("%s: near-tie winner not valid at %s" % (name, bad[:5].tolist()))
    return dict(compared=int(safe.sum()), excluded=int((~safe).sum()))


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


def _close(name, got, ref, rel, abs_=0.0):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = np.abs(ref)
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
    K = host_in["tokens"].shape[2]
    _close("log_w_incr", gpu["log_w_incr"], ora["log_w_incr"], REL, abs_lw(K))
    _close("log_norm", gpu["log_norm"], ora["log_norm"], REL, abs_lw(K))
    stats["lw_below_1"] = int((np.abs(ora["log_w_incr"]) < 1).sum())
    _close("ess", gpu["ess"], ora["ess"], REL, 1e-6)
    if tv:
        _close("tv", gpu["tv"], ora["tv"], REL, 1e-6)
    Kb = host_in["target"].shape[2] - 1
    V = int(host_in.get("V", host_in["gumbel"].shape[-1]))
    b = check_bonus("bonus", gpu["bonus"], ora["bonus"], ora["bonus_gap"],
                    host_in["target"][:, :, Kb], host_in["gumbel"],
                    np.broadcast_to(np.asarray(host_in["temperature"])[:, None],
                                    gpu["bonus"].shape), V)
    stats.update(bonus_compared=b["compared"], bonus_excluded=b["excluded"])

    R = gpu["ancestors"].shape[0]
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
            _close("log_weights[%d]" % r, gpu["log_weights"][r], lw_ref, REL, 2 * abs_lw(K))
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
