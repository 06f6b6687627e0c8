"""CPU reference ("oracle") of one SMC-SD round, in double precision.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline leg of the
benchmark call it to check the GPU library; the library itself never imports it. The
arithmetic lives in ``smcsd_oracle.c`` (plain C, fp64, one loop per definition); this module
only builds that file with gcc and marshals numpy arrays to it.

bf16 arrays are passed as their raw 16-bit patterns (numpy ``uint16``), fp32 as ``float32``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "smcsd_oracle.c")
_SO = os.path.join(_HERE, "libsmcsd_oracle.so")

F32, BF16 = 0, 1
ALWAYS, ESS, NEVER = 0, 1, 2
MODES = {"always": ALWAYS, "ess": ESS, "never": NEVER}

_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP over independent rows, strict IEEE double)."""
    if not force and os.path.exists(_SO):
        return _SO
    tmp = _SO + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _SO)
    return _SO


def lib() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
                build()
            L = ctypes.CDLL(_SO)
            p, i32, i64, f64, f32 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                     ctypes.c_double, ctypes.c_float)
            L.orc_row_logsumexp.restype = f64
            L.orc_row_logsumexp.argtypes = [p, i32, i64, f64]
            L.orc_row_tv.restype = f64
            L.orc_row_tv.argtypes = [p, p, i32, i64, f64]
            L.orc_row_gumbel_argmax.restype = i32
            L.orc_row_gumbel_argmax.argtypes = [p, i32, p, i64, f32, p]
            L.orc_resample_request.restype = i32
            L.orc_resample_request.argtypes = [i32, p, p, f64, i32, f64, p, p, p, p, p]
            L.orc_remap_request.restype = i32
            L.orc_remap_request.argtypes = [i32, i32, p, p, p, p, i32]
            L.orc_round.restype = i32
            L.orc_round.argtypes = [i32, i32, i32, i64, i64, i32, p, p, p, p, p, p, i32, f32, p,
                                    p, p, p, p, p, p, p, p, p, i32, i32, p, p, p, p, p, p]
            L.orc_sd_verify.restype = None
            L.orc_sd_verify.argtypes = [i32, i32, i32, i64, i64, i32, p, p, p, p, p, p, p, p,
                                        p, p, p, p, p]
            L.orc_gumbel_topk.restype = None
            L.orc_gumbel_topk.argtypes = [i64, i64, i64, i32, p, p, p, i32, p, p, p]
            L.orc_bonus_resampled.restype = i32
            L.orc_bonus_resampled.argtypes = [i32, i32, i32, i64, i64, i32, p, p, p, p, p, p]
            L.orc_pages_advance.restype = i32
            L.orc_pages_advance.argtypes = [i32, i32, i32, i32, p, p, p, i32, p, p, p, p, i64, i32,
                                            i32]
            L.orc_num_threads.restype = i32
            L.orc_num_threads.argtypes = []
            _lib = L
    return _lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _logits(z: np.ndarray):
    z = np.ascontiguousarray(z)
    if z.dtype == np.float32:
        return z, F32
    if z.dtype == np.uint16:
        return z, BF16
    raise TypeError("logits must be float32 or raw bf16 bits (uint16), got %s" % z.dtype)


def num_threads() -> int:
    return int(lib().orc_num_threads())


def row_logsumexp(z: np.ndarray, T: float) -> float:
    """log sum_v exp(z_v / T) of one row (fp32 or bf16 bits)."""
    z, dt = _logits(z.reshape(-1))
    return float(lib().orc_row_logsumexp(_ptr(z), dt, z.size, float(T)))


def row_tv(zp: np.ndarray, zq: np.ndarray, T: float) -> float:
    """1/2 sum |p - q| of the temperature-scaled softmaxes of two rows."""
    zp, dt = _logits(zp.reshape(-1))
    zq, dt2 = _logits(zq.reshape(-1))
    assert dt == dt2 and zp.size == zq.size
    return float(lib().orc_row_tv(_ptr(zp), _ptr(zq), dt, zp.size, float(T)))


def row_gumbel_argmax(z: np.ndarray, g: np.ndarray, T: float) -> tuple[int, float]:
    """(argmax_v z_v/T + g_v with keys in double, top-2 key gap)."""
    z, dt = _logits(z.reshape(-1))
    g = np.ascontiguousarray(g.reshape(-1), dtype=np.float32)
    assert g.size == z.size
    gap = np.zeros(1, np.float64)
    idx = lib().orc_row_gumbel_argmax(_ptr(z), dt, _ptr(g), z.size, float(T), _ptr(gap))
    return int(idx), float(gap[0])


def resample_request(lw, logw_prev, u: float, mode="always", ess_frac: float = 0.5):
    """Normalise + ESS + systematic resampling of one request. Returns a dict."""
    lw = np.ascontiguousarray(lw, dtype=np.float64)
    prev = np.ascontiguousarray(logw_prev, dtype=np.float64)
    N = lw.size
    logZ = np.zeros(1)
    ess = np.zeros(1)
    anc = np.zeros(N, np.int32)
    new = np.zeros(N)
    gap = np.zeros(N)
    m = MODES[mode] if isinstance(mode, str) else int(mode)
    rs = lib().orc_resample_request(N, _ptr(lw), _ptr(prev), float(u), m, float(ess_frac),
                                    _ptr(logZ), _ptr(ess), _ptr(anc), _ptr(new), _ptr(gap))
    return dict(resampled=int(rs), log_norm=float(logZ[0]), ess=float(ess[0]), ancestors=anc,
                log_weights=new, anc_gap=gap)


def remap_request(anc, page_table, refcount):
    """Page-table remap of one request. Returns (new table, new refcount, status)."""
    anc = np.ascontiguousarray(anc, dtype=np.int32)
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    N, P = pt.shape
    out = np.zeros_like(pt)
    rc = np.array(refcount, dtype=np.int32, copy=True)
    st = lib().orc_remap_request(N, P, _ptr(anc), _ptr(pt), _ptr(out), _ptr(rc), rc.size)
    return out, rc, int(st)


def round(inputs: dict, *, V: int | None = None, mode="always", ess_frac: float = 0.5,
          tv: bool = False, with_pages: bool = True) -> dict:
    """One full SMC-SD round on host arrays.

    ``inputs`` holds numpy arrays: target [R,N,K+1,ld], draft [R,N,K,ld] (float32 or bf16
    bits as uint16), tokens [R,N,K] int32, temperature [R], gumbel [R,N,ld], uniform [R],
    log_weights [R,N] float32 and optionally page_table [R,N,P] int32 + refcount
    [num_pages] int32, and optionally log_potential [R,N] float32 (log phi added to each
    particle's incremental log weight). ``V`` defaults to ld.
    """
    tgt, dt = _logits(inputs["target"])
    dft, dt2 = _logits(inputs["draft"])
    if dt != dt2:
        raise TypeError("target and draft dtypes differ")
    R, N, K1, ld = tgt.shape
    K = K1 - 1
    if dft.shape != (R, N, K, ld):
        raise ValueError("draft shape %s != %s" % (dft.shape, (R, N, K, ld)))
    V = ld if V is None else int(V)
    tok = np.ascontiguousarray(inputs["tokens"], dtype=np.int32)
    temp = np.ascontiguousarray(inputs["temperature"], dtype=np.float32)
    gum = np.ascontiguousarray(inputs["gumbel"], dtype=np.float32)
    uni = np.ascontiguousarray(inputs["uniform"], dtype=np.float32)
    lwin = np.ascontiguousarray(inputs["log_weights"], dtype=np.float32)
    assert tok.shape == (R, N, K) and temp.shape == (R,) and gum.shape == (R, N, ld)
    assert uni.shape == (R,) and lwin.shape == (R, N)
    lpot = inputs.get("log_potential")
    if lpot is not None:
        lpot = np.ascontiguousarray(lpot, dtype=np.float32)
        assert lpot.shape == (R, N)
    out = dict(
        log_w_incr=np.zeros((R, N)), log_weights=np.zeros((R, N)), log_norm=np.zeros(R),
        ess=np.zeros(R), resampled=np.zeros(R, np.int32), ancestors=np.zeros((R, N), np.int32),
        bonus=np.zeros((R, N), np.int32), out_tokens=np.zeros((R, N, K + 1), np.int32),
        anc_gap=np.zeros((R, N)), bonus_gap=np.zeros((R, N)),
    )
    out["tv"] = np.zeros((R, N, K)) if tv else None
    pt = rc = pt_out = None
    P = num_pages = 0
    if with_pages and inputs.get("page_table") is not None:
        pt = np.ascontiguousarray(inputs["page_table"], dtype=np.int32)
        P = pt.shape[2]
        rc = np.array(inputs["refcount"], dtype=np.int32, copy=True)
        num_pages = rc.size
        pt_out = np.zeros_like(pt)
    m = MODES[mode] if isinstance(mode, str) else int(mode)
    st = lib().orc_round(R, N, K, V, ld, dt, _ptr(tgt), _ptr(dft), _ptr(tok), _ptr(temp),
                         _ptr(gum), _ptr(uni), m, float(ess_frac), _ptr(lwin),
                         _ptr(out["log_w_incr"]), _ptr(out["log_weights"]), _ptr(out["log_norm"]),
                         _ptr(out["ess"]), _ptr(out["resampled"]), _ptr(out["ancestors"]),
                         _ptr(out["bonus"]), _ptr(out["out_tokens"]), _ptr(out["tv"]),
                         P, num_pages, _ptr(pt), _ptr(pt_out), _ptr(rc), _ptr(out["anc_gap"]),
                         _ptr(out["bonus_gap"]), _ptr(lpot))
    out["status"] = int(st)
    out["page_table"] = pt_out
    out["refcount"] = rc
    return out


def sd_verify(inputs: dict, *, V: int | None = None) -> dict:
    """Standard speculative-decoding verification of every particle's drafted tokens.

    ``inputs`` as for ``round`` plus accept_uniform [R,N,K] and residual_uniform [R,N]
    float32. Returns n_accepted [R,N], next_token [R,N] (int32), acc_gap [R,N] (distance
    of the acceptance uniforms from min(1, p/q)), bonus_gap [R,N] (top-2 key gap of the
    bonus draw where the whole block was accepted, +inf elsewhere), and for residual draws
    res_lo / res_hi
    [R,N] (distances of the target from the chosen token's cumulative-sum boundaries, as
    fractions of the residual mass) with res_below / res_above [R,N] (the neighbouring
    tokens with positive residual, -1 if none).
    """
    tgt, dt = _logits(inputs["target"])
    dft, _ = _logits(inputs["draft"])
    R, N, K1, ld = tgt.shape
    K = K1 - 1
    V = ld if V is None else int(V)
    tok = np.ascontiguousarray(inputs["tokens"], dtype=np.int32)
    temp = np.ascontiguousarray(inputs["temperature"], dtype=np.float32)
    gum = np.ascontiguousarray(inputs["gumbel"], dtype=np.float32)
    au = np.ascontiguousarray(inputs["accept_uniform"], dtype=np.float32)
    bu = np.ascontiguousarray(inputs["residual_uniform"], dtype=np.float32)
    assert au.shape == (R, N, K) and bu.shape == (R, N)
    out = dict(n_accepted=np.zeros((R, N), np.int32), next_token=np.zeros((R, N), np.int32),
               acc_gap=np.zeros((R, N)), bonus_gap=np.zeros((R, N)))
    res = np.zeros((R, N, 2))
    nb = np.zeros((R, N, 2), np.int32)
    lib().orc_sd_verify(R, N, K, V, ld, dt, _ptr(tgt), _ptr(dft), _ptr(tok), _ptr(temp),
                        _ptr(gum), _ptr(au), _ptr(bu), _ptr(out["n_accepted"]),
                        _ptr(out["next_token"]), _ptr(out["acc_gap"]), _ptr(res), _ptr(nb),
                        _ptr(out["bonus_gap"]))
    out["res_lo"], out["res_hi"] = res[..., 0], res[..., 1]
    out["res_below"], out["res_above"] = nb[..., 0], nb[..., 1]
    out["res_gap"] = np.minimum(out["res_lo"], out["res_hi"])
    return out


def gumbel_topk(logits: np.ndarray, temperature: np.ndarray, gumbel: np.ndarray, k: int, *,
                V: int | None = None, gaps: bool = False):
    """Gumbel-Top-K of every row: logits [rows, ld] (float32 or bf16 bits as uint16),
    temperature [rows], gumbel [rows, ld] float32. Returns tokens [rows, k] int32 and keys
    [rows, k] float64 (z/T + G in double), in decreasing key order (equal keys by increasing
    index); with gaps=True also gaps [rows, k], key_j - key_(j+1) (+inf past the last token
    of the row)."""
    z, dt = _logits(logits)
    rows, ld = z.shape
    V = ld if V is None else int(V)
    if not 1 <= k <= V:
        raise ValueError("k must be in [1, V]")
    temp = np.ascontiguousarray(temperature, dtype=np.float32)
    g = np.ascontiguousarray(gumbel, dtype=np.float32)
    assert temp.shape == (rows,) and g.shape == (rows, ld)
    tok = np.zeros((rows, k), np.int32)
    key = np.zeros((rows, k), np.float64)
    gap = np.zeros((rows, k), np.float64)
    lib().orc_gumbel_topk(rows, V, ld, dt, _ptr(z), _ptr(temp), _ptr(g), int(k), _ptr(tok),
                          _ptr(key), _ptr(gap))
    return (tok, key, gap) if gaps else (tok, key)


def bonus_resampled(target: np.ndarray, temperature: np.ndarray, ancestors: np.ndarray,
                    gumbel: np.ndarray, *, V: int | None = None) -> dict:
    """Bonus token per new slot after resampling: slot j of request r takes the Gumbel-max
    of its ancestor's target row K with noise row gumbel[r, j]. target [R,N,K+1,ld]
    (float32 or bf16 bits as uint16), temperature [R], ancestors [R,N] int32, gumbel
    [R,N,ld] float32. Returns dict(bonus [R,N] int32, gap [R,N], status)."""
    tgt, dt = _logits(target)
    R, N, K1, ld = tgt.shape
    V = ld if V is None else int(V)
    temp = np.ascontiguousarray(temperature, dtype=np.float32)
    anc = np.ascontiguousarray(ancestors, dtype=np.int32)
    g = np.ascontiguousarray(gumbel, dtype=np.float32)
    assert temp.shape == (R,) and anc.shape == (R, N) and g.shape == (R, N, ld)
    bonus = np.zeros((R, N), np.int32)
    gap = np.zeros((R, N))
    st = lib().orc_bonus_resampled(R, N, K1 - 1, V, ld, dt, _ptr(tgt), _ptr(temp), _ptr(anc),
                                   _ptr(g), _ptr(bonus), _ptr(gap))
    return dict(bonus=bonus, gap=gap, status=int(st))


def pages_advance(page_table: np.ndarray, refcount: np.ndarray, free_ids: np.ndarray,
                  n_free: int, len_before, len_after, page_size: int,
                  kv: np.ndarray | None = None, kv_inplace: bool = False,
                  token_rows: bool = False) -> dict:
    """Page lifecycle between rounds (release at refcount 0, copy-on-write of shared tail
    pages, fresh pages for new columns) on copies of the given host arrays. page_table
    [R,N,P] int32, refcount and free_ids [num_pages] int32, kv uint8 [num_pages, page_bytes]
    or [kv_count, num_pages, page_bytes] (one tensor per layer and K / V) or None; with
    kv_inplace the (C-contiguous uint8) kv array itself receives the copies. token_rows: a
    page is page_size token rows in token order, and a copy moves only the rows the tail
    holds.
    Lengths satisfy 0 <= len_before <= len_after <= P * page_size.
    Returns dict(page_table, refcount, free_ids, n_free, kv, status)."""
    pt = np.array(page_table, dtype=np.int32, copy=True)
    rc = np.array(refcount, dtype=np.int32, copy=True)
    fl = np.array(free_ids, dtype=np.int32, copy=True)
    R, N, P = pt.shape
    lb = np.ascontiguousarray(len_before, dtype=np.int32)
    la = np.ascontiguousarray(len_after, dtype=np.int32)
    assert lb.shape == (R,) and la.shape == (R,)
    assert page_size >= 1 and (lb >= 0).all() and (lb <= la).all() and (la <= P * page_size).all()
    assert fl.size == rc.size and 0 <= n_free <= fl.size
    if kv is None:
        kvc = np.zeros((1, rc.size, 1), np.uint8)
    else:
        if kv_inplace:
            assert kv.dtype == np.uint8 and kv.flags.c_contiguous
            kvc = kv
        else:
            kvc = np.array(kv, dtype=np.uint8, copy=True)
        if kvc.ndim == 2:
            kvc = kvc[None]
        assert kvc.ndim == 3 and kvc.shape[1] == rc.size
        assert not token_rows or kvc.shape[2] % page_size == 0
    nf = np.array([n_free], np.int32)
    st = lib().orc_pages_advance(R, N, P, int(page_size), _ptr(lb), _ptr(la), _ptr(pt), rc.size,
                                 _ptr(rc), _ptr(fl), _ptr(nf), _ptr(kvc), kvc.shape[2],
                                 kvc.shape[0], int(bool(token_rows)))
    if kv is not None and np.ndim(kv) == 2:
        kvc = kvc[0]
    return dict(page_table=pt, refcount=rc, free_ids=fl, n_free=int(nf[0]),
                kv=None if kv is None else kvc, status=int(st))
