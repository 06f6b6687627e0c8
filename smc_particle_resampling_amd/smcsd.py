"""ctypes binding of libsmcsd.so (include/smcsd.h), with the same names as the C entry points.

Argument marshalling only: torch tensors are checked for device, dtype, shape and
contiguity, then their device pointers and the current HIP stream go to the C ABI. Every
step of the round runs in the library's HIP kernels. There is no fallback: importing this
module raises if the library has not been built (``python -m
smc_particle_resampling_amd.build``).
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsmcsd.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError("libsmcsd.so is not built (expected at %s); run "
                      "`python -m smc_particle_resampling_amd.build`" % _LIB_PATH)
_lib = ctypes.CDLL(_LIB_PATH)

OK, ERR_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_DEVICE, ERR_SCRATCH = 0, 1, 2, 3, 4, 5
NOALLOC_SCRATCH_BYTES = 16 << 20
F32, BF16 = 0, 1
RESAMPLE_ALWAYS, RESAMPLE_ESS, RESAMPLE_NEVER = 0, 1, 2
MODES = {"always": RESAMPLE_ALWAYS, "ess": RESAMPLE_ESS, "never": RESAMPLE_NEVER}
DEVERR_TOKEN, DEVERR_ANCESTOR, DEVERR_PAGE, DEVERR_REFCOUNT, DEVERR_EXCHANGE = 1, 2, 4, 8, 16
DEVERR_POOL, DEVERR_LENGTH = 32, 64
MAX_N, MAX_K = 1024, 256

_i32, _i64, _f32, _p, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t


class RoundArgs(ctypes.Structure):
    """Mirror of smcsd_round_args."""
    _fields_ = [
        ("R", _i32), ("N", _i32), ("K", _i32), ("V", _i32), ("ld", _i64), ("dtype", _i32),
        ("mode", _i32), ("ess_frac", _f32), ("P", _i32), ("num_pages", _i32), ("reserved0", _i32),
        ("target_logits", _p), ("draft_logits", _p), ("draft_tokens", _p), ("temperature", _p),
        ("gumbel", _p), ("uniform", _p), ("log_weights", _p), ("log_w_incr", _p),
        ("log_norm", _p), ("ess", _p), ("resampled", _p), ("ancestors", _p), ("bonus", _p),
        ("out_tokens", _p), ("tv", _p), ("page_table_in", _p), ("page_table_out", _p),
        ("refcount", _p), ("error_flags", _p), ("workspace", _p), ("workspace_bytes", _sz),
        ("timing_begin", _p), ("timing_end", _p), ("log_potential", _p), ("timing_split", _p),
    ]


class VerifyArgs(ctypes.Structure):
    """Mirror of smcsd_verify_args."""
    _fields_ = [
        ("R", _i32), ("N", _i32), ("K", _i32), ("V", _i32), ("ld", _i64), ("dtype", _i32),
        ("reserved0", _i32),
        ("target_logits", _p), ("draft_logits", _p), ("draft_tokens", _p), ("temperature", _p),
        ("gumbel", _p), ("accept_uniform", _p), ("residual_uniform", _p),
        ("n_accepted", _p), ("next_token", _p), ("tv", _p), ("error_flags", _p),
        ("workspace", _p), ("workspace_bytes", _sz), ("timing_begin", _p), ("timing_end", _p),
    ]


_lib.smcsd_round.restype = _i32
_lib.smcsd_round.argtypes = [ctypes.POINTER(RoundArgs), _p]
_lib.smcsd_round_noalloc.restype = _i32
_lib.smcsd_round_noalloc.argtypes = [ctypes.POINTER(RoundArgs), _p]
_lib.smcsd_resample.restype = _i32
_lib.smcsd_resample.argtypes = [_i32, _i32, _p, _p, _p, _i32, _f32, _p, _p, _p, _p, _p]
_lib.smcsd_remap_pages.restype = _i32
_lib.smcsd_remap_pages.argtypes = [_i32, _i32, _i32, _p, _p, _p, _p, _i32, _p, _p]
_lib.smcsd_workspace_size.restype = _sz
_lib.smcsd_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32]
_lib.smcsd_status_string.restype = ctypes.c_char_p
_lib.smcsd_status_string.argtypes = [_i32]
_lib.smcsd_round_args_size.restype = _sz
_lib.smcsd_round_args_size.argtypes = []
_lib.smcsd_sd_verify.restype = _i32
_lib.smcsd_sd_verify.argtypes = [ctypes.POINTER(VerifyArgs), _p]
_lib.smcsd_verify_workspace_size.restype = _sz
_lib.smcsd_verify_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32]
_lib.smcsd_verify_args_size.restype = _sz
_lib.smcsd_verify_args_size.argtypes = []
_lib.smcsd_gumbel_topk.restype = _i32
_lib.smcsd_gumbel_topk.argtypes = [_i32, _i32, _i64, _i32, _p, _p, _p, _i32, _p, _p, _p, _sz, _p]
_lib.smcsd_topk_workspace_size.restype = _sz
_lib.smcsd_topk_workspace_size.argtypes = [_i32, _i32, _i32, _i32]
_lib.smcsd_bench_stream_read.restype = _i32
_lib.smcsd_bonus_resampled.restype = _i32
_lib.smcsd_bonus_resampled.argtypes = [_i32, _i32, _i32, _i32, _i64, _i32, _p, _p, _p, _p, _p, _p,
                                       _p, _sz, _p, _p]
_lib.smcsd_bonus_workspace_size.restype = _sz
_lib.smcsd_bonus_workspace_size.argtypes = [_i32, _i32, _i32, _i32]
_lib.smcsd_pages_advance.restype = _i32
_lib.smcsd_pages_advance.argtypes = [_i32, _i32, _i32, _i32, _p, _p, _p, _i32, _p, _p, _p, _p,
                                     _i64, _i32, _i64, _i32, _p, _sz, _p, _p, _p]
_lib.smcsd_pages_workspace_size.restype = _sz
_lib.smcsd_pages_workspace_size.argtypes = [_i32, _i32, _i32, _i32]
_lib.smcsd_bench_stream_read.argtypes = [_p, _sz, _p, _i32, _p]
_lib.smcsd_bench_copy.restype = _i32
_lib.smcsd_bench_copy.argtypes = [_p, _p, _sz, _p]
_lib.smcsd_bench_logits_pass.restype = _i32
_lib.smcsd_bench_logits_pass.argtypes = [ctypes.c_void_p, _i32, _p]


class SmcsdError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__("%s: %s (status %d)" % (where, smcsd_status_string(status), status))
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def raw_library() -> ctypes.CDLL:
    return _lib


def smcsd_status_string(status: int) -> str:
    return _lib.smcsd_status_string(int(status)).decode()


def smcsd_round_args_size() -> int:
    return int(_lib.smcsd_round_args_size())


MAX_TOPK = 64


def smcsd_topk_workspace_size(rows: int, V: int, dtype: int, k: int) -> int:
    return int(_lib.smcsd_topk_workspace_size(rows, V, dtype, k))


def smcsd_verify_args_size() -> int:
    return int(_lib.smcsd_verify_args_size())


def smcsd_verify_workspace_size(R: int, N: int, K: int, V: int, dtype: int) -> int:
    return int(_lib.smcsd_verify_workspace_size(R, N, K, V, dtype))


def smcsd_workspace_size(R: int, N: int, K: int, V: int, dtype: int, tv_enabled: bool) -> int:
    return int(_lib.smcsd_workspace_size(R, N, K, V, dtype, int(bool(tv_enabled))))


# ------------------------------------------------------------------ marshalling helpers
def _ptr(t: torch.Tensor | None):
    return None if t is None else t.data_ptr()


def _check(t, name, dtype, shape, device):
    if t is None:
        raise ValueError("%s is required" % name)
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _stream(device, stream):
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return torch.cuda.current_stream(device).cuda_stream


def smcsd_round(*, workspace, stream=None, **kw) -> None:
    """Enqueue one SMC-SD round (smcsd_round). Shapes: target [R,N,K+1,ld], draft
    [R,N,K,ld] (both float32 or bfloat16), draft_tokens [R,N,K] int32, temperature [R],
    gumbel [R,N,ld], uniform [R], per-request/per-particle outputs as in include/smcsd.h;
    workspace a uint8 device tensor of at least smcsd_workspace_size() bytes."""
    a, dev = _round_args(workspace=workspace, **kw)
    st = _lib.smcsd_round(ctypes.byref(a), _stream(dev, stream))
    if st != OK:
        raise SmcsdError(st, "smcsd_round")


class RoundCall:
    """One smcsd_round whose arguments are checked and marshalled once: launch() enqueues the
    same round again (the tensors' contents may change between launches, not their shapes or
    storage). For callers, such as a benchmark loop, whose per-call host overhead would
    otherwise exceed a small round's GPU time. Same keyword arguments as smcsd_round."""

    def __init__(self, *, stream=None, noalloc=False, **kw):
        self._keep = kw                       # the tensors stay alive with the call
        ws = None if noalloc else kw.pop("workspace")
        self._args, dev = _round_args(workspace=ws, **kw)
        self._ref = ctypes.byref(self._args)
        self._stream = _stream(dev, stream)
        self._fn = _lib.smcsd_round_noalloc if noalloc else _lib.smcsd_round

    def bench_pass(self, repeats: int) -> None:
        """Enqueue the round's logits pass alone, `repeats` times (smcsd_bench_logits_pass)."""
        if self._fn is not _lib.smcsd_round:
            raise ValueError("bench_pass needs a round with a workspace")
        a = self._args
        a.timing_begin = a.timing_split = a.timing_end = None
        st = _lib.smcsd_bench_logits_pass(self._ref, int(repeats), self._stream)
        if st != OK:
            raise SmcsdError(st, "smcsd_bench_logits_pass")

    def launch(self, timing_events=None) -> None:
        a = self._args
        a.timing_begin = a.timing_split = a.timing_end = None
        if timing_events is not None:
            if len(timing_events) == 3:
                a.timing_begin, a.timing_split, a.timing_end = timing_events
            else:
                a.timing_begin, a.timing_end = timing_events
        st = self._fn(self._ref, self._stream)
        if st != OK:
            raise SmcsdError(st, "smcsd_round")


def smcsd_round_noalloc(*, stream=None, **kw) -> None:
    """smcsd_round without a workspace argument (smcsd_round_noalloc): the library's static
    per-GPU scratch buffer serves as the workspace, and the call allocates nothing. Same
    arguments as smcsd_round except ``workspace``."""
    a, dev = _round_args(workspace=None, **kw)
    st = _lib.smcsd_round_noalloc(ctypes.byref(a), _stream(dev, stream))
    if st != OK:
        raise SmcsdError(st, "smcsd_round_noalloc")


def _round_args(*, target_logits, draft_logits, draft_tokens, temperature, gumbel, uniform,
                log_weights, log_w_incr, log_norm, ess, resampled, ancestors, bonus,
                workspace, out_tokens=None, tv=None, page_table_in=None, page_table_out=None,
                refcount=None, error_flags=None, log_potential=None, V: int | None = None,
                mode="always", ess_frac: float = 0.5, timing_events=None):
    """The smcsd_round_args struct of a round, after checking every tensor."""
    dev = target_logits.device
    if target_logits.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("logits must be float32 or bfloat16")
    if target_logits.dim() != 4:
        raise ValueError("target_logits must be [R, N, K+1, ld]")
    R, N, K1, ld = target_logits.shape
    K = K1 - 1
    V = ld if V is None else int(V)
    f32, i32 = torch.float32, torch.int32
    _check(target_logits, "target_logits", None, None, dev)
    _check(draft_logits, "draft_logits", target_logits.dtype, (R, N, K, ld), dev)
    _check(draft_tokens, "draft_tokens", i32, (R, N, K), dev)
    _check(temperature, "temperature", f32, (R,), dev)
    if gumbel is not None:                     # None: no bonus inside the round
        _check(gumbel, "gumbel", f32, (R, N, ld), dev)
    _check(uniform, "uniform", f32, (R,), dev)
    _check(log_weights, "log_weights", f32, (R, N), dev)
    _check(log_w_incr, "log_w_incr", f32, (R, N), dev)
    _check(log_norm, "log_norm", f32, (R,), dev)
    _check(ess, "ess", f32, (R,), dev)
    _check(resampled, "resampled", i32, (R,), dev)
    _check(ancestors, "ancestors", i32, (R, N), dev)
    if bonus is not None or gumbel is not None:
        _check(bonus, "bonus", i32, (R, N), dev)
    if workspace is not None:
        _check(workspace, "workspace", torch.uint8, None, dev)
    if out_tokens is not None:
        _check(out_tokens, "out_tokens", i32, (R, N, K + 1), dev)
    if tv is not None:
        _check(tv, "tv", f32, (R, N, K), dev)
    P = num_pages = 0
    if page_table_in is not None:
        P = page_table_in.shape[-1]
        _check(page_table_in, "page_table_in", i32, (R, N, P), dev)
        _check(page_table_out, "page_table_out", i32, (R, N, P), dev)
        _check(refcount, "refcount", i32, None, dev)
        num_pages = refcount.numel()
    if error_flags is not None:
        _check(error_flags, "error_flags", i32, None, dev)
    if log_potential is not None:
        _check(log_potential, "log_potential", f32, (R, N), dev)
    a = RoundArgs()
    a.R, a.N, a.K, a.V, a.ld = R, N, K, V, ld
    a.dtype = BF16 if target_logits.dtype == torch.bfloat16 else F32
    a.mode = MODES[mode] if isinstance(mode, str) else int(mode)
    a.ess_frac = float(ess_frac)
    a.P, a.num_pages, a.reserved0 = P, num_pages, 0
    a.target_logits, a.draft_logits = _ptr(target_logits), _ptr(draft_logits)
    a.draft_tokens, a.temperature = _ptr(draft_tokens), _ptr(temperature)
    a.gumbel, a.uniform, a.log_weights = _ptr(gumbel), _ptr(uniform), _ptr(log_weights)
    a.log_w_incr, a.log_norm, a.ess = _ptr(log_w_incr), _ptr(log_norm), _ptr(ess)
    a.resampled, a.ancestors, a.bonus = _ptr(resampled), _ptr(ancestors), _ptr(bonus)
    a.out_tokens, a.tv = _ptr(out_tokens), _ptr(tv)
    a.page_table_in, a.page_table_out = _ptr(page_table_in), _ptr(page_table_out)
    a.refcount, a.error_flags = _ptr(refcount), _ptr(error_flags)
    a.log_potential = _ptr(log_potential)
    a.workspace, a.workspace_bytes = _ptr(workspace), (0 if workspace is None else workspace.numel())
    if timing_events is not None:
        # (begin, end) around the logits pass, or (begin, split, end): split also separates
        # the row-pair kernel from the bonus-row kernel of a TV pass
        if len(timing_events) == 3:
            a.timing_begin, a.timing_split, a.timing_end = timing_events
        else:
            a.timing_begin, a.timing_end = timing_events
    return a, dev


def smcsd_sd_verify(*, target_logits, draft_logits, draft_tokens, temperature, gumbel,
                    accept_uniform, residual_uniform, n_accepted, next_token, workspace, tv=None,
                    error_flags=None, V: int | None = None, timing_events=None,
                    stream=None) -> None:
    """Enqueue standard speculative-decoding verification (smcsd_sd_verify) of every
    particle's drafted block. Shapes as for smcsd_round plus accept_uniform [R,N,K] and
    residual_uniform [R,N] float32; outputs n_accepted, next_token [R,N] int32."""
    dev = target_logits.device
    if target_logits.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("logits must be float32 or bfloat16")
    if target_logits.dim() != 4:
        raise ValueError("target_logits must be [R, N, K+1, ld]")
    R, N, K1, ld = target_logits.shape
    K = K1 - 1
    V = ld if V is None else int(V)
    f32, i32 = torch.float32, torch.int32
    _check(target_logits, "target_logits", None, None, dev)
    _check(draft_logits, "draft_logits", target_logits.dtype, (R, N, K, ld), dev)
    _check(draft_tokens, "draft_tokens", i32, (R, N, K), dev)
    _check(temperature, "temperature", f32, (R,), dev)
    _check(gumbel, "gumbel", f32, (R, N, ld), dev)
    _check(accept_uniform, "accept_uniform", f32, (R, N, K), dev)
    _check(residual_uniform, "residual_uniform", f32, (R, N), dev)
    _check(n_accepted, "n_accepted", i32, (R, N), dev)
    _check(next_token, "next_token", i32, (R, N), dev)
    _check(workspace, "workspace", torch.uint8, None, dev)
    if tv is not None:
        _check(tv, "tv", f32, (R, N, K), dev)
    if error_flags is not None:
        _check(error_flags, "error_flags", i32, None, dev)
    a = VerifyArgs()
    a.R, a.N, a.K, a.V, a.ld = R, N, K, V, ld
    a.dtype = BF16 if target_logits.dtype == torch.bfloat16 else F32
    a.reserved0 = 0
    a.target_logits, a.draft_logits = _ptr(target_logits), _ptr(draft_logits)
    a.draft_tokens, a.temperature, a.gumbel = _ptr(draft_tokens), _ptr(temperature), _ptr(gumbel)
    a.accept_uniform, a.residual_uniform = _ptr(accept_uniform), _ptr(residual_uniform)
    a.n_accepted, a.next_token, a.tv = _ptr(n_accepted), _ptr(next_token), _ptr(tv)
    a.error_flags = _ptr(error_flags)
    a.workspace, a.workspace_bytes = _ptr(workspace), workspace.numel()
    if timing_events is not None:
        a.timing_begin, a.timing_end = timing_events
    st = _lib.smcsd_sd_verify(ctypes.byref(a), _stream(dev, stream))
    if st != OK:
        raise SmcsdError(st, "smcsd_sd_verify")


def smcsd_gumbel_topk(*, logits, temperature, gumbel, k: int, out_tokens, workspace,
                      out_keys=None, V: int | None = None, stream=None) -> None:
    """Enqueue Gumbel-Top-K (smcsd_gumbel_topk): logits [rows, ld] float32/bfloat16,
    temperature [rows], gumbel [rows, ld] float32 -> out_tokens [rows, k] int32 (and
    out_keys [rows, k] float32), by decreasing key."""
    dev = logits.device
    if logits.dtype not in (torch.float32, torch.bfloat16) or logits.dim() != 2:
        raise ValueError("logits must be a [rows, ld] float32 or bfloat16 tensor")
    rows, ld = logits.shape
    V = ld if V is None else int(V)
    f32, i32 = torch.float32, torch.int32
    _check(logits, "logits", None, None, dev)
    _check(temperature, "temperature", f32, (rows,), dev)
    _check(gumbel, "gumbel", f32, (rows, ld), dev)
    _check(out_tokens, "out_tokens", i32, (rows, k), dev)
    if out_keys is not None:
        _check(out_keys, "out_keys", f32, (rows, k), dev)
    _check(workspace, "workspace", torch.uint8, None, dev)
    dt = BF16 if logits.dtype == torch.bfloat16 else F32
    st = _lib.smcsd_gumbel_topk(rows, V, ld, dt, _ptr(logits), _ptr(temperature), _ptr(gumbel),
                                int(k), _ptr(out_tokens), _ptr(out_keys), _ptr(workspace),
                                workspace.numel(), _stream(dev, stream))
    if st != OK:
        raise SmcsdError(st, "smcsd_gumbel_topk")


def gumbel_topk(logits, temperature, gumbel, k: int, *, V: int | None = None, outputs=None,
                stream=None) -> dict:
    """smcsd_gumbel_topk with outputs and workspace allocated here (or reused from
    ``outputs``). Returns dict(tokens, keys, workspace)."""
    rows, ld = logits.shape
    V = ld if V is None else int(V)
    dev = logits.device
    if outputs is None:
        dt = BF16 if logits.dtype == torch.bfloat16 else F32
        ws = smcsd_topk_workspace_size(rows, V, dt, k)
        if ws == 0 and rows > 0:
            raise ValueError("sizes unsupported: rows=%d V=%d k=%d" % (rows, V, k))
        outputs = dict(tokens=torch.empty((rows, k), dtype=torch.int32, device=dev),
                       keys=torch.empty((rows, k), dtype=torch.float32, device=dev),
                       workspace=torch.empty((max(ws, 256),), dtype=torch.uint8, device=dev))
    smcsd_gumbel_topk(logits=logits, temperature=temperature, gumbel=gumbel, k=k,
                      out_tokens=outputs["tokens"], out_keys=outputs["keys"],
                      workspace=outputs["workspace"], V=V, stream=stream)
    return outputs


def smcsd_resample(*, log_w_incr, log_weights, uniform, log_norm, ess, resampled, ancestors,
                   mode="always", ess_frac: float = 0.5, stream=None) -> None:
    """Enqueue normalise + ESS + systematic resampling from given log-weight increments."""
    dev = log_w_incr.device
    R, N = log_w_incr.shape
    f32, i32 = torch.float32, torch.int32
    _check(log_w_incr, "log_w_incr", f32, (R, N), dev)
    _check(log_weights, "log_weights", f32, (R, N), dev)
    _check(uniform, "uniform", f32, (R,), dev)
    _check(log_norm, "log_norm", f32, (R,), dev)
    _check(ess, "ess", f32, (R,), dev)
    _check(resampled, "resampled", i32, (R,), dev)
    _check(ancestors, "ancestors", i32, (R, N), dev)
    m = MODES[mode] if isinstance(mode, str) else int(mode)
    st = _lib.smcsd_resample(R, N, _ptr(log_w_incr), _ptr(log_weights), _ptr(uniform), m,
                             float(ess_frac), _ptr(log_norm), _ptr(ess), _ptr(resampled),
                             _ptr(ancestors), _stream(dev, stream))
    if st != OK:
        raise SmcsdError(st, "smcsd_resample")


def smcsd_remap_pages(*, ancestors, page_table_in, page_table_out, refcount, error_flags=None,
                      stream=None) -> None:
    """Enqueue the page-table remap by pointer exchange."""
    dev = ancestors.device
    R, N, P = page_table_in.shape
    i32 = torch.int32
    _check(ancestors, "ancestors", i32, (R, N), dev)
    _check(page_table_in, "page_table_in", i32, (R, N, P), dev)
    _check(page_table_out, "page_table_out", i32, (R, N, P), dev)
    _check(refcount, "refcount", i32, None, dev)
    if error_flags is not None:
        _check(error_flags, "error_flags", i32, None, dev)
    st = _lib.smcsd_remap_pages(R, N, P, _ptr(ancestors), _ptr(page_table_in),
                                _ptr(page_table_out), _ptr(refcount), refcount.numel(),
                                _ptr(error_flags), _stream(dev, stream))
    if st != OK:
        raise SmcsdError(st, "smcsd_remap_pages")


def smcsd_bonus_workspace_size(R: int, N: int, V: int, dtype: int) -> int:
    return int(_lib.smcsd_bonus_workspace_size(R, N, V, dtype))


def smcsd_bonus_resampled(*, target_logits, temperature, ancestors, gumbel, bonus, workspace,
                          out_tokens=None, error_flags=None, V: int | None = None,
                          stream=None) -> None:
    """Enqueue the bonus draw after resampling (smcsd_bonus_resampled): slot j of request r
    takes the Gumbel-max of its ancestor's target row K with noise row gumbel[r, j]. Shapes:
    target [R,N,K+1,ld], temperature [R], ancestors [R,N], gumbel [R,N,ld], bonus [R,N],
    out_tokens None or [R,N,K+1] (column K receives the bonus)."""
    dev = target_logits.device
    if target_logits.dtype not in (torch.float32, torch.bfloat16) or target_logits.dim() != 4:
        raise ValueError("target_logits must be float32 or bfloat16 [R, N, K+1, ld]")
    R, N, K1, ld = target_logits.shape
    V = ld if V is None else int(V)
    f32, i32 = torch.float32, torch.int32
    _check(target_logits, "target_logits", None, None, dev)
    _check(temperature, "temperature", f32, (R,), dev)
    _check(ancestors, "ancestors", i32, (R, N), dev)
    _check(gumbel, "gumbel", f32, (R, N, ld), dev)
    _check(bonus, "bonus", i32, (R, N), dev)
    _check(workspace, "workspace", torch.uint8, None, dev)
    if out_tokens is not None:
        _check(out_tokens, "out_tokens", i32, (R, N, K1), dev)
    if error_flags is not None:
        _check(error_flags, "error_flags", i32, None, dev)
    dt = BF16 if target_logits.dtype == torch.bfloat16 else F32
    st = _lib.smcsd_bonus_resampled(R, N, K1 - 1, V, ld, dt, _ptr(target_logits),
                                    _ptr(temperature), _ptr(ancestors), _ptr(gumbel),
                                    _ptr(bonus), _ptr(out_tokens), _ptr(workspace),
                                    workspace.numel(), _ptr(error_flags), _stream(dev, stream))
    if st != OK:
        raise SmcsdError(st, "smcsd_bonus_resampled")


def smcsd_pages_workspace_size(R: int, N: int, P: int, num_pages: int) -> int:
    return int(_lib.smcsd_pages_workspace_size(R, N, P, num_pages))


def smcsd_pages_advance(*, len_before, len_after, page_table, refcount, free_ids, n_free,
                        page_size: int, workspace, kv=None, token_rows: bool = False,
                        stats=None, error_flags=None, stream=None) -> None:
    """Enqueue the page lifecycle between rounds (smcsd_pages_advance). page_table [R,N,P],
    len_before / len_after [R], refcount / free_ids [num_pages], n_free [1], all int32; kv
    None or a uint8 tensor [num_pages, page_bytes] or [kv_count, num_pages, page_bytes];
    token_rows: token-major pages, copy only the tail's filled rows."""
    dev = page_table.device
    R, N, P = page_table.shape
    i32 = torch.int32
    _check(page_table, "page_table", i32, (R, N, P), dev)
    _check(len_before, "len_before", i32, (R,), dev)
    _check(len_after, "len_after", i32, (R,), dev)
    _check(refcount, "refcount", i32, None, dev)
    num_pages = refcount.numel()
    _check(free_ids, "free_ids", i32, (num_pages,), dev)
    _check(n_free, "n_free", i32, (1,), dev)
    _check(workspace, "workspace", torch.uint8, None, dev)
    page_bytes, kv_count, kv_stride = 0, 0, 0
    if kv is not None:
        _check(kv, "kv", torch.uint8, None, dev)
        if kv.dim() == 2:
            kv_count, page_bytes = 1, kv.shape[1]
        elif kv.dim() == 3:
            kv_count, page_bytes = kv.shape[0], kv.shape[2]
        else:
            raise ValueError("kv must be [num_pages, page_bytes] or [kv_count, num_pages, page_bytes]")
        if kv.shape[-2] != num_pages:
            raise ValueError("kv holds %d pages, refcount %d" % (kv.shape[-2], num_pages))
        kv_stride = num_pages * page_bytes
    if stats is not None:
        _check(stats, "stats", i32, (5,), dev)
    if error_flags is not None:
        _check(error_flags, "error_flags", i32, None, dev)
    st = _lib.smcsd_pages_advance(R, N, P, int(page_size), _ptr(len_before), _ptr(len_after),
                                  _ptr(page_table), num_pages, _ptr(refcount), _ptr(free_ids),
                                  _ptr(n_free), _ptr(kv), page_bytes, kv_count, kv_stride,
                                  int(bool(token_rows)), _ptr(workspace), workspace.numel(),
                                  _ptr(stats),
                                  _ptr(error_flags), _stream(dev, stream))
    if st != OK:
        raise SmcsdError(st, "smcsd_pages_advance")


def smcsd_bench_stream_read(src: torch.Tensor, sink: torch.Tensor, grid: int, stream=None) -> None:
    st = _lib.smcsd_bench_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                                      int(grid), _stream(src.device, stream))
    if st != OK:
        raise SmcsdError(st, "smcsd_bench_stream_read")


def smcsd_bench_copy(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    st = _lib.smcsd_bench_copy(_ptr(src), _ptr(dst), src.numel() * src.element_size(),
                               _stream(src.device, stream))
    if st != OK:
        raise SmcsdError(st, "smcsd_bench_copy")


# ------------------------------------------------------------------ allocation conveniences
def alloc_outputs(R: int, N: int, K: int, device, tv: bool = False, out_tokens: bool = True,
                  V: int = 1, dtype: int = BF16) -> dict:
    """Output tensors and a workspace for smcsd_round (torch allocates; nothing is computed)."""
    f32, i32 = torch.float32, torch.int32
    ws = smcsd_workspace_size(R, N, K, V, dtype, tv)
    if ws == 0 and R > 0:
        raise ValueError("sizes unsupported: R=%d N=%d K=%d V=%d" % (R, N, K, V))
    return dict(
        log_w_incr=torch.empty((R, N), dtype=f32, device=device),
        log_norm=torch.empty((R,), dtype=f32, device=device),
        ess=torch.empty((R,), dtype=f32, device=device),
        resampled=torch.empty((R,), dtype=i32, device=device),
        ancestors=torch.empty((R, N), dtype=i32, device=device),
        bonus=torch.empty((R, N), dtype=i32, device=device),
        out_tokens=torch.empty((R, N, K + 1), dtype=i32, device=device) if out_tokens else None,
        tv=torch.empty((R, N, K), dtype=f32, device=device) if tv else None,
        error_flags=torch.zeros((1,), dtype=i32, device=device),
        workspace=torch.empty((max(ws, 256),), dtype=torch.uint8, device=device),
    )


def run_round(inputs: dict, *, mode="always", ess_frac=0.5, tv=False, pages=True, outputs=None,
              timing_events=None, bonus_noise=None, stream=None) -> dict:
    """smcsd_round on a dict from ``synth.make_inputs`` (log_weights, page tables and refcount
    are updated in place / swapped like a caller would). Returns the output tensors.
    With ``bonus_noise`` ([R,N,ld] float32) the round draws no bonus itself; the bonus is
    drawn after resampling, per new slot, with that noise (smcsd_bonus_resampled)."""
    tgt = inputs["target"]
    R, N, K1, ld = tgt.shape
    K = K1 - 1
    dt = BF16 if tgt.dtype == torch.bfloat16 else F32
    out = outputs or alloc_outputs(R, N, K, tgt.device, tv=tv, V=inputs["V"], dtype=dt)
    pt_in = inputs.get("page_table") if pages else None
    if pt_in is not None and "page_table_out" not in out:
        out["page_table_out"] = torch.empty_like(pt_in)
    after = bonus_noise is not None
    smcsd_round(target_logits=tgt, draft_logits=inputs["draft"], draft_tokens=inputs["tokens"],
                temperature=inputs["temperature"], gumbel=None if after else inputs["gumbel"],
                uniform=inputs["uniform"], log_weights=inputs["log_weights"],
                log_w_incr=out["log_w_incr"], log_norm=out["log_norm"], ess=out["ess"],
                resampled=out["resampled"], ancestors=out["ancestors"], bonus=out["bonus"],
                out_tokens=out.get("out_tokens"), tv=out.get("tv"), page_table_in=pt_in,
                page_table_out=out.get("page_table_out") if pt_in is not None else None,
                refcount=inputs.get("refcount") if pt_in is not None else None,
                error_flags=out["error_flags"], workspace=out["workspace"],
                log_potential=inputs.get("log_potential"), V=inputs["V"],
                mode=mode, ess_frac=ess_frac, timing_events=timing_events, stream=stream)
    if after:
        if "bonus_workspace" not in out:
            ws = smcsd_bonus_workspace_size(R, N, inputs["V"], dt)
            out["bonus_workspace"] = torch.empty((max(ws, 256),), dtype=torch.uint8,
                                                 device=tgt.device)
        smcsd_bonus_resampled(target_logits=tgt, temperature=inputs["temperature"],
                              ancestors=out["ancestors"], gumbel=bonus_noise,
                              bonus=out["bonus"], out_tokens=out.get("out_tokens"),
                              workspace=out["bonus_workspace"], error_flags=out["error_flags"],
                              V=inputs["V"], stream=stream)
    return out


def run_sd_verify(inputs: dict, *, tv=False, outputs=None, timing_events=None, stream=None) -> dict:
    """smcsd_sd_verify on a dict from ``synth.make_inputs`` that also holds accept_uniform
    and residual_uniform (``synth.make_verify_uniforms``). Returns the output tensors."""
    tgt = inputs["target"]
    R, N, K1, ld = tgt.shape
    K = K1 - 1
    dev = tgt.device
    dt = BF16 if tgt.dtype == torch.bfloat16 else F32
    if outputs is None:
        ws = smcsd_verify_workspace_size(R, N, K, inputs["V"], dt)
        if ws == 0 and R > 0:
            raise ValueError("sizes unsupported: R=%d N=%d K=%d V=%d" % (R, N, K, inputs["V"]))
        outputs = dict(
            n_accepted=torch.empty((R, N), dtype=torch.int32, device=dev),
            next_token=torch.empty((R, N), dtype=torch.int32, device=dev),
            tv=torch.empty((R, N, K), dtype=torch.float32, device=dev) if tv else None,
            error_flags=torch.zeros((1,), dtype=torch.int32, device=dev),
            workspace=torch.empty((max(ws, 256),), dtype=torch.uint8, device=dev))
    o = outputs
    smcsd_sd_verify(target_logits=tgt, draft_logits=inputs["draft"], draft_tokens=inputs["tokens"],
                    temperature=inputs["temperature"], gumbel=inputs["gumbel"],
                    accept_uniform=inputs["accept_uniform"],
                    residual_uniform=inputs["residual_uniform"], n_accepted=o["n_accepted"],
                    next_token=o["next_token"], workspace=o["workspace"], tv=o.get("tv"),
                    error_flags=o["error_flags"], V=inputs["V"], timing_events=timing_events,
                    stream=stream)
    return o


__all__ = [n for n in dir() if n.startswith("smcsd_")] + [
    "RoundArgs", "VerifyArgs", "SmcsdError", "alloc_outputs", "run_round", "run_sd_verify",
    "gumbel_topk", "library_path", "MODES", "MAX_TOPK"]
