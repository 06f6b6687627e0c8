"""C-ABI checks that need no GPU: the library loads, exports every function include/*.h
declares, the binding's struct layout matches, and host-side argument validation returns
the documented status codes before any HIP call."""
import ctypes
import os
import re

import pytest

from smc_particle_resampling_amd import smcsd as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in ("smcsd.h", "smcsd_bench.h"):
        src = open(os.path.join(ROOT, "include", h)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*(smcsd_[A-Za-z0-9_]+)\s*\(",
                             src, flags=re.M):
            names.add(m.group(1))
    return names


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert {"smcsd_round", "smcsd_resample", "smcsd_remap_pages", "smcsd_workspace_size",
            "smcsd_status_string", "smcsd_round_args_size", "smcsd_bench_stream_read",
            "smcsd_bench_copy", "smcsd_bench_logits_pass", "smcsd_sd_verify",
            "smcsd_verify_workspace_size",
            "smcsd_verify_args_size", "smcsd_gumbel_topk", "smcsd_topk_workspace_size",
            "smcsd_pages_advance", "smcsd_pages_workspace_size", "smcsd_bonus_resampled",
            "smcsd_bonus_workspace_size", "smcsd_round_noalloc"} <= names
    lib = ctypes.CDLL(S.library_path())
    for n in sorted(names):
        assert hasattr(lib, n), n


def test_struct_layout_matches():
    assert S.smcsd_verify_args_size() == ctypes.sizeof(S.VerifyArgs)
    assert S.VerifyArgs.target_logits.offset == 32
    assert S.smcsd_round_args_size() == ctypes.sizeof(S.RoundArgs)
    assert S.RoundArgs.ld.offset == 16
    assert S.RoundArgs.target_logits.offset == 48


def test_status_strings():
    for st in range(6):
        assert S.smcsd_status_string(st) not in ("", "unknown status")
    assert S.smcsd_status_string(99) == "unknown status"


def test_workspace_size():
    a = S.smcsd_workspace_size(64, 32, 8, 128256, S.BF16, True)
    b = S.smcsd_workspace_size(64, 32, 8, 128256, S.BF16, False)
    assert a > b > 0 and a % 256 == 0
    assert S.smcsd_workspace_size(1, 0, 4, 100, S.BF16, False) == 0          # N = 0
    assert S.smcsd_workspace_size(1, 8, 0, 100, S.BF16, False) == 0          # K = 0
    assert S.smcsd_workspace_size(1, 8, 4, 100, 7, False) == 0               # dtype
    assert S.smcsd_workspace_size(1, S.MAX_N + 1, 4, 100, S.BF16, False) == 0


# A syntactically valid argument block with fake, aligned, non-null device pointers. The
# calls below must fail validation before touching them.
def _args(**kw):
    a = S.RoundArgs()
    a.R, a.N, a.K, a.V, a.ld = 2, 8, 4, 1000, 1000
    a.dtype, a.mode, a.ess_frac = S.BF16, S.RESAMPLE_ALWAYS, 0.5
    base = 0x10000000
    for i, (name, _) in enumerate(S.RoundArgs._fields_[11:30]):
        setattr(a, name, base + 0x100000 * i)
    a.page_table_in = None
    a.workspace = base + 0x8000000
    a.workspace_bytes = 1 << 30
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _round(a):
    return S.raw_library().smcsd_round(ctypes.byref(a), None)


@pytest.mark.parametrize("field,value,status", [
    ("N", 0, S.ERR_ARG), ("K", 0, S.ERR_ARG), ("V", 0, S.ERR_ARG), ("R", -1, S.ERR_ARG),
    ("ld", 999, S.ERR_ARG), ("ld", 1004, S.ERR_ARG), ("dtype", 2, S.ERR_ARG),
    ("mode", 3, S.ERR_ARG), ("reserved0", 1, S.ERR_ARG),
    ("N", S.MAX_N + 1, S.ERR_UNSUPPORTED), ("K", S.MAX_K + 1, S.ERR_UNSUPPORTED),
    ("target_logits", None, S.ERR_ARG), ("draft_logits", None, S.ERR_ARG),
    ("draft_tokens", None, S.ERR_ARG), ("gumbel", 0x10000008, S.ERR_ARG),  # misaligned
    ("uniform", None, S.ERR_ARG),
    ("log_weights", None, S.ERR_ARG), ("ancestors", None, S.ERR_ARG), ("bonus", None, S.ERR_ARG),
    ("target_logits", 0x10000008, S.ERR_ARG),                # not 16-byte aligned
    ("workspace", None, S.ERR_WORKSPACE), ("workspace_bytes", 100, S.ERR_WORKSPACE),
    ("workspace", 0x18000010, S.ERR_WORKSPACE),              # not 256-byte aligned
])
def test_round_validation(field, value, status):
    assert _round(_args(**{field: value})) == status


def test_round_validation_ess_and_pages():
    assert _round(_args(mode=S.RESAMPLE_ESS, ess_frac=0.0)) == S.ERR_ARG
    assert _round(_args(mode=S.RESAMPLE_ESS, ess_frac=1.5)) == S.ERR_ARG
    pt = 0x30000000
    assert _round(_args(page_table_in=pt, page_table_out=pt, P=4, num_pages=10)) == S.ERR_ARG
    assert _round(_args(page_table_in=pt, page_table_out=pt + 64, P=4, num_pages=10)) == S.ERR_ARG
    assert _round(_args(page_table_in=pt, page_table_out=None, P=4, num_pages=10)) == S.ERR_ARG
    assert _round(_args(page_table_in=pt, page_table_out=pt + (1 << 20), P=0, num_pages=10)) == S.ERR_ARG
    # TV: at most 64 slices of 512 lanes x 4 chunks (V <= 1048576 bf16, 524288 f32)
    assert _round(_args(V=1048576 + 8, ld=1048576 + 8)) == S.ERR_UNSUPPORTED
    assert _round(_args(V=1048576 + 8, ld=1048576 + 8, tv=None, workspace_bytes=100)) == S.ERR_WORKSPACE
    assert _round(_args(dtype=S.F32, V=524288 + 4, ld=524288 + 4)) == S.ERR_UNSUPPORTED
    # fp32 rows need ld % 4 == 0 only
    assert _round(_args(dtype=S.F32, ld=1004, workspace_bytes=100)) == S.ERR_WORKSPACE


def test_empty_batch_is_a_no_op():
    assert _round(_args(R=0)) == S.OK
    assert _round(_args(R=0, target_logits=None)) == S.OK


def test_noalloc_validation():
    """smcsd_round_noalloc validates on the host like smcsd_round, refuses a workspace of the
    caller's, and refuses a request larger than its static scratch buffer, all before any
    HIP call."""
    lib = S.raw_library()

    def call(a):
        return lib.smcsd_round_noalloc(ctypes.byref(a), None)

    hdr = open(os.path.join(ROOT, "include", "smcsd.h")).read()
    m = re.search(r"SMCSD_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", hdr)
    assert int(m.group(1)) << int(m.group(2)) == S.NOALLOC_SCRATCH_BYTES
    none = dict(workspace=None, workspace_bytes=0)
    assert call(_args()) == S.ERR_ARG                                   # a workspace given
    assert call(_args(workspace=None)) == S.ERR_ARG                     # ... or its size
    assert call(_args(N=0, **none)) == S.ERR_ARG
    assert call(_args(V=1048576 + 8, ld=1048576 + 8, **none)) == S.ERR_UNSUPPORTED
    assert call(_args(R=0, **none)) == S.OK
    big = dict(R=512, N=32, K=8, V=128256, ld=128256)
    need = S.smcsd_workspace_size(512, 32, 8, 128256, S.BF16, True)
    assert need > S.NOALLOC_SCRATCH_BYTES
    assert call(_args(**big, **none)) == S.ERR_SCRATCH
    assert S.smcsd_workspace_size(64, 32, 8, 128256, S.BF16, True) <= S.NOALLOC_SCRATCH_BYTES
    assert S.smcsd_workspace_size(32, 32, 8, 256000, S.BF16, True) <= S.NOALLOC_SCRATCH_BYTES


def test_resample_and_remap_validation():
    lib = S.raw_library()
    p = 0x10000000
    assert lib.smcsd_resample(1, 0, p, p, p, 0, 0.5, p, p, p, p, None) == S.ERR_ARG
    assert lib.smcsd_resample(1, 4, None, p, p, 0, 0.5, p, p, p, p, None) == S.ERR_ARG
    assert lib.smcsd_resample(1, 4, p, p, p, 5, 0.5, p, p, p, p, None) == S.ERR_ARG
    assert lib.smcsd_resample(1, 4, p, p, p, 1, 0.0, p, p, p, p, None) == S.ERR_ARG
    assert lib.smcsd_resample(1, S.MAX_N + 1, p, p, p, 0, 0.5, p, p, p, p, None) == S.ERR_UNSUPPORTED
    assert lib.smcsd_resample(0, 4, None, None, None, 0, 0.5, None, None, None, None, None) == S.OK
    assert lib.smcsd_remap_pages(1, 4, 0, p, p, p + 4096, p, 10, None, None) == S.ERR_ARG
    assert lib.smcsd_remap_pages(1, 4, 4, p, p, p, p, 10, None, None) == S.ERR_ARG     # alias
    assert lib.smcsd_remap_pages(1, 4, 4, None, p, p + 4096, p, 10, None, None) == S.ERR_ARG
    assert lib.smcsd_remap_pages(0, 4, 4, None, None, None, None, 10, None, None) == S.OK
    assert lib.smcsd_bench_copy(p, p, 64, None) == S.ERR_ARG
    assert lib.smcsd_bench_stream_read(p + 4, 64, p, 1, None) == S.ERR_ARG
    assert lib.smcsd_bench_logits_pass(None, 1, None) == S.ERR_ARG
    a = S.RoundArgs()
    assert lib.smcsd_bench_logits_pass(ctypes.byref(a), 0, None) == S.ERR_ARG      # repeats


def test_binding_rejects_bad_tensors_before_the_library():
    import torch
    t = torch.zeros(1, 2, 3, 8)
    with pytest.raises(ValueError):
        S.smcsd_round(target_logits=t.to(torch.float16), draft_logits=None, draft_tokens=None,
                      temperature=None, gumbel=None, uniform=None, log_weights=None,
                      log_w_incr=None, log_norm=None, ess=None, resampled=None, ancestors=None,
                      bonus=None, workspace=None)
    with pytest.raises(ValueError):
        S.smcsd_round(target_logits=t, draft_logits=torch.zeros(1, 2, 3, 8), draft_tokens=None,
                      temperature=None, gumbel=None, uniform=None, log_weights=None,
                      log_w_incr=None, log_norm=None, ess=None, resampled=None, ancestors=None,
                      bonus=None, workspace=None)


def _vargs(**kw):
    a = S.VerifyArgs()
    a.R, a.N, a.K, a.V, a.ld, a.dtype = 2, 8, 4, 1000, 1000, S.BF16
    base = 0x20000000
    for i, name in enumerate(("target_logits", "draft_logits", "draft_tokens", "temperature",
                              "gumbel", "accept_uniform", "residual_uniform", "n_accepted",
                              "next_token")):
        setattr(a, name, base + i * (1 << 24))
    a.workspace = 0x70000000
    a.workspace_bytes = S.smcsd_verify_workspace_size(2, 8, 4, 1000, S.BF16)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _verify(a):
    return S.raw_library().smcsd_sd_verify(ctypes.byref(a), None)


def test_verify_validation():
    ws = S.smcsd_verify_workspace_size(2, 8, 4, 1000, S.BF16)
    assert ws > 0 and ws % 256 == 0
    assert ws > S.smcsd_workspace_size(2, 8, 4, 1000, S.BF16, True)
    assert _verify(_vargs(R=0)) == S.OK
    assert _verify(_vargs(N=0)) == S.ERR_ARG
    assert _verify(_vargs(reserved0=1)) == S.ERR_ARG
    assert _verify(_vargs(ld=1001)) == S.ERR_ARG
    assert _verify(_vargs(accept_uniform=None)) == S.ERR_ARG
    assert _verify(_vargs(residual_uniform=None)) == S.ERR_ARG
    assert _verify(_vargs(next_token=None)) == S.ERR_ARG
    assert _verify(_vargs(target_logits=0x20000008)) == S.ERR_ARG
    assert _verify(_vargs(N=S.MAX_N + 1)) == S.ERR_UNSUPPORTED
    assert _verify(_vargs(workspace_bytes=100)) == S.ERR_WORKSPACE
    assert _verify(_vargs(workspace=0x70000010)) == S.ERR_WORKSPACE
    # TV is always on here: V beyond the TV limit is unsupported
    big = 1048576 + 8
    assert _verify(_vargs(V=big, ld=big)) == S.ERR_UNSUPPORTED


def _topk(rows=4, V=1000, ld=1000, dtype=S.BF16, logits=0x20000000, temperature=0x21000000,
          gumbel=0x22000000, k=8, out_tokens=0x23000000, ws=0x70000000, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = S.smcsd_topk_workspace_size(max(rows, 0), V, dtype, max(k, 1))
    return S.raw_library().smcsd_gumbel_topk(rows, V, ld, dtype, logits, temperature, gumbel, k,
                                             out_tokens, None, ws, ws_bytes, None)


def test_topk_validation():
    assert S.smcsd_topk_workspace_size(4, 1000, S.BF16, 8) > 0
    assert S.smcsd_topk_workspace_size(4, 1000, S.BF16, 0) == 0
    assert S.smcsd_topk_workspace_size(4, 1000, S.BF16, S.MAX_TOPK + 1) == 0
    assert S.smcsd_topk_workspace_size(4, 10, S.BF16, 11) == 0              # k > V
    assert _topk(rows=0) == S.OK
    assert _topk(k=0) == S.ERR_ARG
    assert _topk(k=S.MAX_TOPK + 1) == S.ERR_UNSUPPORTED
    assert _topk(V=10, ld=16, k=11) == S.ERR_ARG                              # k > V
    assert _topk(ld=1004) == S.ERR_ARG                                        # bf16 ld % 8
    assert _topk(logits=None) == S.ERR_ARG
    assert _topk(gumbel=0x22000004) == S.ERR_ARG                              # alignment
    assert _topk(ws_bytes=16) == S.ERR_WORKSPACE
    assert _topk(ws=0x70000010) == S.ERR_WORKSPACE
    big = 1048576 + 8
    assert _topk(V=big, ld=big) == S.ERR_UNSUPPORTED                         # > 64 slices


def test_pages_workspace_size():
    a = S.smcsd_pages_workspace_size(64, 32, 64, 100000)
    assert a > 0 and a % 256 == 0
    assert S.smcsd_pages_workspace_size(64, 32, 64, 200000) > a            # more chunks
    assert S.smcsd_pages_workspace_size(0, 32, 64, 100) > 0                # release only
    assert S.smcsd_pages_workspace_size(1, 0, 64, 100) == 0
    assert S.smcsd_pages_workspace_size(1, 8, 64, 0) == 0
    assert S.smcsd_pages_workspace_size(1, S.MAX_N + 1, 4, 100) == 0
    assert S.smcsd_pages_workspace_size(4096, 1024, 1024, 100) == 0        # R*N*P >= 2^31


def _pages(**kw):
    base = 0x10000000
    a = dict(R=2, N=4, P=8, page_size=16, len_before=base, len_after=base + 0x1000,
             page_table=base + 0x2000, num_pages=100, refcount=base + 0x10000,
             free_ids=base + 0x20000, n_free=base + 0x30000, kv=None, page_bytes=0,
             kv_count=0, kv_stride=0, token_rows=0, workspace=base + 0x40000,
             workspace_bytes=1 << 20,
             stats=None, error_flags=None)
    a.update(kw)
    return S.raw_library().smcsd_pages_advance(
        a["R"], a["N"], a["P"], a["page_size"], a["len_before"], a["len_after"],
        a["page_table"], a["num_pages"], a["refcount"], a["free_ids"], a["n_free"], a["kv"],
        a["page_bytes"], a["kv_count"], a["kv_stride"], a["token_rows"], a["workspace"],
        a["workspace_bytes"],
        a["stats"], a["error_flags"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(N=0), S.ERR_ARG),
    (dict(R=-1), S.ERR_ARG),
    (dict(P=0), S.ERR_ARG),
    (dict(page_size=0), S.ERR_ARG),
    (dict(num_pages=0), S.ERR_ARG),
    (dict(N=S.MAX_N + 1), S.ERR_UNSUPPORTED),
    (dict(R=4096, N=1024, P=1024), S.ERR_UNSUPPORTED),
    (dict(refcount=None), S.ERR_ARG),
    (dict(free_ids=None), S.ERR_ARG),
    (dict(n_free=None), S.ERR_ARG),
    (dict(len_before=None), S.ERR_ARG),
    (dict(page_table=None), S.ERR_ARG),
    (dict(workspace=None), S.ERR_WORKSPACE),
    (dict(workspace_bytes=64), S.ERR_WORKSPACE),
    (dict(kv=0x50000000, page_bytes=8, kv_count=1), S.ERR_ARG),          # not a multiple of 16
    (dict(kv=0x50000008, page_bytes=64, kv_count=1), S.ERR_ARG),         # misaligned
    (dict(kv=0x50000000, page_bytes=64, kv_count=0), S.ERR_ARG),
    (dict(kv=0x50000000, page_bytes=64, kv_count=2, kv_stride=64 * 99), S.ERR_ARG),  # overlap
    (dict(free_ids=0x10010100), S.ERR_ARG),                              # overlaps refcount
    (dict(n_free=0x10040010), S.ERR_ARG),                                # inside the workspace
    (dict(stats=0x10030000), S.ERR_ARG),                                 # overlaps n_free
    (dict(workspace=0x10040010), S.ERR_WORKSPACE),                       # not 256-byte aligned
    (dict(kv=0x50000000, page_bytes=48, kv_count=1, token_rows=1), S.ERR_ARG),   # 3 B a row
    (dict(kv=0x50000000, page_bytes=16 * 24, kv_count=1, token_rows=1), S.ERR_ARG),  # 24 B rows
])
def test_pages_validation(kw, status):
    assert _pages(**kw) == status


def test_bonus_workspace_size():
    a = S.smcsd_bonus_workspace_size(64, 32, 128256, S.BF16)
    assert a > 0 and a % 256 == 0
    assert a == S.smcsd_topk_workspace_size(64 * 32, 128256, S.BF16, 1)
    assert S.smcsd_bonus_workspace_size(1, 0, 100, S.BF16) == 0
    assert S.smcsd_bonus_workspace_size(1, S.MAX_N + 1, 100, S.BF16) == 0
    assert S.smcsd_bonus_workspace_size(1, 8, 100, 7) == 0


def _bonus(**kw):
    base = 0x10000000
    a = dict(R=2, N=8, K=4, V=1000, ld=1000, dtype=S.BF16, target=base, temperature=base + 0x100000,
             ancestors=base + 0x200000, gumbel=base + 0x300000, bonus=base + 0x400000,
             out_tokens=None, workspace=base + 0x500000, workspace_bytes=1 << 20,
             error_flags=None)
    a.update(kw)
    return S.raw_library().smcsd_bonus_resampled(
        a["R"], a["N"], a["K"], a["V"], a["ld"], a["dtype"], a["target"], a["temperature"],
        a["ancestors"], a["gumbel"], a["bonus"], a["out_tokens"], a["workspace"],
        a["workspace_bytes"], a["error_flags"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(N=0), S.ERR_ARG),
    (dict(K=0), S.ERR_ARG),
    (dict(V=0), S.ERR_ARG),
    (dict(R=-1), S.ERR_ARG),
    (dict(ld=999), S.ERR_ARG),
    (dict(ld=1004), S.ERR_ARG),                 # not a multiple of 8 for bf16
    (dict(dtype=2), S.ERR_ARG),
    (dict(N=S.MAX_N + 1), S.ERR_UNSUPPORTED),
    (dict(K=S.MAX_K + 1), S.ERR_UNSUPPORTED),
    (dict(target=None), S.ERR_ARG),
    (dict(ancestors=None), S.ERR_ARG),
    (dict(gumbel=None), S.ERR_ARG),
    (dict(bonus=None), S.ERR_ARG),
    (dict(gumbel=0x10300008), S.ERR_ARG),       # misaligned
    (dict(workspace=None), S.ERR_WORKSPACE),
    (dict(workspace_bytes=16), S.ERR_WORKSPACE),
    (dict(workspace=0x10500010), S.ERR_WORKSPACE),
])
def test_bonus_validation(kw, status):
    assert _bonus(**kw) == status


def test_empty_bonus_call_is_a_no_op():
    assert _bonus(R=0, target=None, temperature=None, ancestors=None, gumbel=None, bonus=None,
                  workspace=None) == S.OK


def test_round_without_noise_is_still_validated():
    # gumbel NULL (no bonus in the round) is valid, so these calls must fail on another
    # argument before anything is launched.
    assert _round(_args(gumbel=None, bonus=None, uniform=None)) == S.ERR_ARG
    assert _round(_args(gumbel=None, workspace_bytes=100)) == S.ERR_WORKSPACE
    assert _round(_args(gumbel=None, N=S.MAX_N + 1)) == S.ERR_UNSUPPORTED
