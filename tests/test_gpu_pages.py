"""GPU parity of the page lifecycle between rounds (smcsd_pages_advance, through the C ABI)
against the oracle, and of a multi-round driver: SMC-SD rounds in ESS mode, each followed by
the remap and the page lifecycle, with the GPU chain and the oracle chain each carrying its
own state.

The SMC-SD page (section 2) shares KV pages between duplicated particles by page metadata;
the pool around that follows the readings in the oracle's header (release at refcount 0 in
id order, copy-on-write of a shared partly filled tail page, fresh pages for new columns,
stack pops request by request). Everything here is integer or byte work: page tables,
refcounts, the free list, its count and the KV bytes must match bit for bit.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import parity
from smc_particle_resampling_amd import smcsd, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _gpu_advance(pool, dev, lens=None, token_rows=False):
    """Copies the pool to the device, runs smcsd_pages_advance, returns host arrays."""
    R, N, P = pool["page_table"].shape
    lb, la = lens if lens is not None else (pool["len_before"], pool["len_after"])
    t = dict(page_table=pool["page_table"].to(dev), refcount=pool["refcount"].to(dev),
             free_ids=pool["free_ids"].to(dev),
             n_free=torch.tensor([pool["n_free"]], dtype=torch.int32, device=dev),
             len_before=torch.as_tensor(lb, dtype=torch.int32).to(dev),
             len_after=torch.as_tensor(la, dtype=torch.int32).to(dev),
             kv=None if pool.get("kv") is None else pool["kv"].to(dev))
    num_pages = t["refcount"].numel()
    ws = torch.empty(max(256, smcsd.smcsd_pages_workspace_size(R, N, P, num_pages)),
                     dtype=torch.uint8, device=dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    stats = torch.full((5,), -5, dtype=torch.int32, device=dev)
    smcsd.smcsd_pages_advance(page_size=pool["page_size"], workspace=ws, error_flags=flags,
                              stats=stats, token_rows=token_rows, **t)
    torch.cuda.synchronize()
    out = {k: (None if v is None else v.cpu().numpy()) for k, v in t.items()}
    out["n_free"] = int(out["n_free"][0])
    out["flags"] = int(flags.item())
    out["stats"] = stats.cpu().numpy().tolist()
    return out


def _expected_stats(pool, o, lens=None, token_rows=False):
    """[released, pops served, pages copied, pops unserved, token rows copied] read off the
    oracle's result."""
    lb, la = lens if lens is not None else (pool["len_before"], pool["len_after"])
    lb, la = np.asarray(lb, np.int64), np.asarray(la, np.int64)
    ps = pool["page_size"]
    pt0, pt1 = pool["page_table"].numpy(), o["page_table"]
    released = int((pool["refcount"].numpy() == 0).sum())
    served = pool["n_free"] + released - o["n_free"]
    copied = unserved = rows = 0
    for r in range(pt0.shape[0]):
        if lb[r] > 0 and lb[r] % ps:
            c = (lb[r] - 1) // ps
            changed = pt1[r, :, c] != pt0[r, :, c]
            n = int((changed & (pt1[r, :, c] >= 0)).sum())
            copied += n
            rows += n * (int(lb[r] % ps) if token_rows else ps)
            unserved += int((changed & (pt1[r, :, c] < 0)).sum())
        c0, c1 = -(-lb[r] // ps), -(-la[r] // ps)
        unserved += int((pt1[r, :, c0:c1] < 0).sum())
    return [released, served, copied, unserved, rows]


def _oracle_advance(pool, lens=None, token_rows=False):
    lb, la = lens if lens is not None else (pool["len_before"], pool["len_after"])
    kv = pool.get("kv")
    return oracle.pages_advance(pool["page_table"].numpy(), pool["refcount"].numpy(),
                                pool["free_ids"].numpy(), pool["n_free"], np.asarray(lb),
                                np.asarray(la), pool["page_size"],
                                None if kv is None else kv.numpy(), token_rows=token_rows)


def _compare(g, o, expect_flags=0):
    assert g["flags"] == expect_flags, "device error flags %d" % g["flags"]
    for k in ("page_table", "refcount", "free_ids"):
        if not np.array_equal(g[k], o[k]):
            bad = np.argwhere(g[k] != o[k])[:5]
            raise AssertionError("%s differs at %s: gpu %s oracle %s" % (
                k, bad.tolist(), g[k][tuple(bad.T)], o[k][tuple(bad.T)]))
    assert g["n_free"] == o["n_free"]
    if o["kv"] is not None:
        if not np.array_equal(g["kv"], o["kv"]):
            bad = np.argwhere((g["kv"] != o["kv"]).any(axis=-1))[:5]
            raise AssertionError("kv pages differ: %s" % bad.tolist())


def test_hand_worked_case(dev):
    num_pages, page_bytes = 16, 16
    rc = torch.full((num_pages,), -1, dtype=torch.int32)
    free = torch.zeros(num_pages, dtype=torch.int32)
    free[:12] = torch.tensor(list(range(10)) + [14, 15], dtype=torch.int32)
    rc[10], rc[11], rc[12], rc[13] = 3, 2, 1, 0
    kv = torch.arange(num_pages * page_bytes, dtype=torch.int32).to(torch.uint8)
    pool = dict(page_table=torch.tensor([[[10, 11, -1], [10, 11, -1], [10, 12, -1]]],
                                        dtype=torch.int32),
                refcount=rc, free_ids=free, n_free=12, len_before=torch.tensor([6]),
                len_after=torch.tensor([9]), kv=kv.view(1, num_pages, page_bytes), page_size=4)
    g = _gpu_advance(pool, dev)
    assert g["page_table"].tolist() == [[[10, 11, 15], [10, 13, 14], [10, 12, 9]]]
    _compare(g, _oracle_advance(pool))


# (R, N, P, page_size, steps, spare, kv_count, page_bytes, seed)
CASES = [
    (3, 8, 6, 4, None, 40, 2, 32, 1),            # mixed steps, copies and appends
    (8, 32, 16, 16, 9, 400, 4, 256, 2),          # 32 particles, page 16, K + 1 = 9 tokens
    (4, 16, 12, 8, 0, 8, 1, 64, 3),              # no new tokens: copy-on-write only
    (4, 16, 12, 8, 19, 700, 1, 16, 4),           # three new columns per particle
    (3, 12, 20, 1, 3, 200, 0, 0, 5),             # page size 1: tails are always full
    (2, 1, 8, 4, 5, 8, 1, 32, 6),                # one particle: nothing shared
    (2, 37, 9, 5, None, 300, 1, 48, 7),          # ragged particle count
    (2, 1024, 3, 8, 7, 2048, 1, 16, 8),          # particle maximum
    (4, 64, 20, 8, 8, 3000, 0, 0, 9),            # > 4096 pages: several ragged chunks
    (6, 24, 10, 4, None, 0, 1, 32, 10),          # empty free list at entry
    (64, 32, 30, 16, 9, 65536, 2, 64, 14),       # the driver bench's shape: 64 x 32, page 16
]


@pytest.mark.parametrize("case", CASES, ids=["R%d-N%d-P%d-ps%d-s%s-sp%d-kv%d" % c[:7] for c in CASES])
def test_advance_matches_oracle(case, dev):
    R, N, P, ps, steps, spare, kvc, pb, seed = case
    _say("case", case)
    pool = synth.make_page_pool(R, N, P, ps, seed, steps=steps, spare=spare, kv_count=kvc,
                                page_bytes=pb)
    o = _oracle_advance(pool)
    g = _gpu_advance(pool, dev)
    _compare(g, o, expect_flags=smcsd.DEVERR_POOL if o["status"] == -3 else 0)
    assert g["stats"] == _expected_stats(pool, o)
    _say("  ok: status", o["status"], "free", pool["n_free"], "->", o["n_free"], "stats", g["stats"])


# token-major pages: (R, N, P, page_size, steps, spare, kv_count, page_bytes, seed), rows of
# page_bytes / page_size = 16, 16, 16 and 32 bytes
TOKEN_ROW_CASES = [
    (3, 8, 6, 4, None, 40, 2, 64, 1),
    (2, 37, 9, 5, None, 300, 1, 80, 7),
    (6, 24, 10, 4, None, 0, 1, 64, 10),
    (64, 32, 30, 16, 9, 65536, 2, 512, 14),
]


@pytest.mark.parametrize("case", TOKEN_ROW_CASES,
                         ids=["R%d-N%d-P%d-ps%d-s%s-sp%d-kv%d" % c[:7] for c in TOKEN_ROW_CASES])
def test_token_rows_match_oracle(case, dev):
    R, N, P, ps, steps, spare, kvc, pb, seed = case
    _say("case", case)
    pool = synth.make_page_pool(R, N, P, ps, seed, steps=steps, spare=spare, kv_count=kvc,
                                page_bytes=pb)
    o = _oracle_advance(pool, token_rows=True)
    g = _gpu_advance(pool, dev, token_rows=True)
    _compare(g, o, expect_flags=smcsd.DEVERR_POOL if o["status"] == -3 else 0)
    assert g["stats"] == _expected_stats(pool, o, token_rows=True)
    full = _oracle_advance(pool)
    assert np.array_equal(full["page_table"], o["page_table"])
    if g["stats"][2] > 0:
        assert not np.array_equal(full["kv"], o["kv"])      # fewer bytes were copied
    _say("  ok: stats", g["stats"])


def test_free_list_runs_dry(dev):
    # Spare pages cover only part of the pops: the GPU leaves the same entries -1 as the
    # oracle, and flags it.
    pool = synth.make_page_pool(4, 16, 12, 4, 11, steps=17, spare=20, kv_count=1, page_bytes=32)
    o = _oracle_advance(pool)
    assert o["status"] == -3
    g = _gpu_advance(pool, dev)
    _compare(g, o, expect_flags=smcsd.DEVERR_POOL)
    assert g["n_free"] == 0 and o["n_free"] == 0
    assert g["stats"] == _expected_stats(pool, o) and g["stats"][3] > 0


def test_release_only(dev):
    # No requests: only pages at refcount 0 go on the free list, in increasing id, behind
    # the ones already there.
    n = 9000
    g_ = torch.Generator().manual_seed(3)
    rc = torch.randint(-1, 3, (n,), generator=g_).to(torch.int32)
    free_pages = torch.nonzero(rc == -1).flatten().to(torch.int32)
    free = torch.full((n,), -7, dtype=torch.int32)
    free[:free_pages.numel()] = free_pages[torch.randperm(free_pages.numel(), generator=g_)]
    pool = dict(page_table=torch.zeros((0, 4, 3), dtype=torch.int32), refcount=rc,
                free_ids=free, n_free=int(free_pages.numel()), len_before=torch.zeros(0),
                len_after=torch.zeros(0), kv=None, page_size=4)
    g = _gpu_advance(pool, dev)
    _compare(g, _oracle_advance(pool))
    assert g["n_free"] == int((rc <= 0).sum())


def test_bad_lengths_leave_the_request_alone(dev):
    pool = synth.make_page_pool(3, 8, 8, 4, 12, steps=5, spare=100, kv_count=1, page_bytes=16)
    lb = pool["len_before"].clone()
    la = pool["len_after"].clone()
    la[1] = lb[1] - 1                                  # shrinking length: invalid
    g = _gpu_advance(pool, dev, lens=(lb, la))
    # The oracle with request 1 doing nothing (lengths 0, 0) is what the GPU must produce.
    lb0, la0 = lb.clone(), la.clone()
    lb0[1] = la0[1] = 0
    _compare(g, _oracle_advance(pool, lens=(lb0, la0)), expect_flags=smcsd.DEVERR_LENGTH)
    assert np.array_equal(g["page_table"][1], pool["page_table"][1].numpy())


def test_repeated_calls_are_identical(dev):
    pool = synth.make_page_pool(8, 32, 16, 16, 13, steps=9, spare=500, kv_count=2,
                                page_bytes=128)
    a = _gpu_advance(pool, dev)
    b = _gpu_advance(pool, dev)
    for k in ("page_table", "refcount", "free_ids", "kv"):
        assert np.array_equal(a[k], b[k]), k


# ---------------------------------------------------------------- multi-round driver
def _host(t):
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


@pytest.mark.parametrize("mode,rounds,seed,token_rows", [("ess", 6, 21, False),
                                                        ("always", 4, 22, False),
                                                        ("ess", 5, 23, True)])
def test_multi_round_driver(mode, rounds, seed, token_rows, dev):
    """Rounds of propose -> weight -> resample (ESS-adaptive) -> remap -> page lifecycle.
    The GPU chain and the oracle chain start from the same seeded state and each carries its
    own log-weights, page table, refcounts, free list and KV bytes; every round compares them."""
    w = synth.WORKLOADS["r16-n16-k4-v128256-bf16"].scaled(
        name="driver", R=3, N=16, K=3, V=6000, mode=mode, ess_frac=0.5)
    K, ps, P = w.K, 4, 16
    pool = synth.make_page_pool(w.R, w.N, P, ps, seed, steps=rounds * (K + 1), spare=400,
                                kv_count=2, page_bytes=64, min_len=2)
    base = synth.make_inputs(w, seed, device=dev, pages=False)
    # GPU state
    g_lw = base["log_weights"].clone()
    g_pt = pool["page_table"].to(dev)
    g_rc = pool["refcount"].to(dev)
    g_free = pool["free_ids"].to(dev)
    g_nfree = torch.tensor([pool["n_free"]], dtype=torch.int32, device=dev)
    g_kv = pool["kv"].to(dev)
    # oracle state
    o_lw = _host(base["log_weights"]).astype(np.float32)
    o_pt, o_rc = pool["page_table"].numpy().copy(), pool["refcount"].numpy().copy()
    o_free, o_nfree, o_kv = pool["free_ids"].numpy().copy(), pool["n_free"], pool["kv"].numpy().copy()
    length = pool["len_before"].clone()
    ws = torch.empty(smcsd.smcsd_pages_workspace_size(w.R, w.N, P, g_rc.numel()),
                     dtype=torch.uint8, device=dev)
    resampled_rounds = 0
    for t in range(rounds):
        _say("round", t, "mode", mode, "lengths", length.tolist())
        fresh = synth.make_inputs(w, 1000 * seed + t, device=dev, pages=False)
        inp = dict(fresh, log_weights=g_lw, page_table=g_pt, refcount=g_rc)
        out = smcsd.run_round(inp, mode=mode, ess_frac=w.ess_frac)
        remapped = out["page_table_out"].clone()           # before the lifecycle changes it
        lb = length.to(torch.int32)
        la = (length + K + 1).to(torch.int32)
        smcsd.smcsd_pages_advance(len_before=lb.to(dev), len_after=la.to(dev),
                                  page_table=out["page_table_out"], refcount=g_rc,
                                  free_ids=g_free, n_free=g_nfree, page_size=ps, workspace=ws,
                                  kv=g_kv, token_rows=token_rows, error_flags=out["error_flags"])
        torch.cuda.synchronize()
        assert int(out["error_flags"].item()) == 0

        host = {k: _host(fresh[k]) for k in ("target", "draft", "tokens", "temperature",
                                             "gumbel", "uniform")}
        host.update(log_weights=o_lw, page_table=o_pt, refcount=o_rc, V=w.V)
        ora = oracle.round(host, V=w.V, mode=mode, ess_frac=w.ess_frac)
        assert ora["status"] == 0
        # The chains stay comparable only without near ties; the seeds are chosen so.
        assert np.all(ora["anc_gap"] >= parity.ANC_GAP), "near tie: pick another seed"
        if mode == "ess":
            assert np.all(np.abs(ora["ess"] - w.ess_frac * w.N) >= 1e-4 * w.N), "ESS at threshold"
        anc = out["ancestors"].cpu().numpy()
        assert np.array_equal(anc, ora["ancestors"])
        assert np.array_equal(out["resampled"].cpu().numpy(), ora["resampled"])
        gb = out["bonus"].cpu().numpy()
        parity.check_bonus("bonus", gb, ora["bonus"], ora["bonus_gap"], host["target"][:, :, w.K],
                           host["gumbel"], np.broadcast_to(host["temperature"][:, None], gb.shape),
                           w.V)
        parity._close("log_weights", g_lw.cpu().numpy(), ora["log_weights"], parity.REL,
                      2 * parity.abs_lw(w.K))
        assert np.array_equal(remapped.cpu().numpy(), ora["page_table"])
        resampled_rounds += int(ora["resampled"].sum())

        adv = oracle.pages_advance(ora["page_table"], ora["refcount"], o_free, o_nfree,
                                   lb.numpy(), la.numpy(), ps, o_kv, token_rows=token_rows)
        assert adv["status"] == 0
        g = dict(page_table=out["page_table_out"].cpu().numpy(), refcount=g_rc.cpu().numpy(),
                 free_ids=g_free.cpu().numpy(), n_free=int(g_nfree.item()),
                 kv=g_kv.cpu().numpy(), flags=0)
        _compare(g, adv)
        # carry both chains
        g_pt = out["page_table_out"]
        o_lw = ora["log_weights"].astype(np.float32)
        o_pt, o_rc, o_free, o_nfree, o_kv = (adv["page_table"], adv["refcount"],
                                            adv["free_ids"], adv["n_free"], adv["kv"])
        length = length + K + 1
        _say("  ok: resampled", ora["resampled"].tolist(), "free", o_nfree)
    assert resampled_rounds > 0
