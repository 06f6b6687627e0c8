"""GPU parity: the HIP round (through the C ABI) against the CPU oracle on the same seeded
inputs, element by element, to the bar in tests/parity.py.

Sizes: every workload scaled down so the oracle finishes in seconds while still spanning
several slices per row and a ragged last chunk; every workload at full size, every request
compared; and the edge cases (V = 1, V not a multiple of 8, N = 1, N at its maximum, K = 1,
empty batch, p == q, every resample mode, masked vocabulary ranges, out-of-range ids).
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import parity
from smc_particle_resampling_amd import smcsd, synth

pytestmark = pytest.mark.gpu
W = synth.WORKLOADS


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_and_compare(w: synth.Workload, dev, seed=0, requests=None, pages=True, ragged=False,
                    inputs=None, modify=None):
    _say("case", w.name, "R N K V", w.R, w.N, w.K, w.V, "ld", w.row_stride, "seed", seed,
         "requests", requests)
    inp = inputs or synth.make_inputs(w, seed, device=dev, ragged_pages=ragged)
    if modify:
        modify(inp)
    host = synth.to_host(inp, requests)
    rc_before = inp["refcount"].cpu().numpy().copy() if pages else None
    out = smcsd.run_round(inp, mode=w.mode, ess_frac=w.ess_frac, tv=w.tv, pages=pages)
    torch.cuda.synchronize()
    assert int(out["error_flags"].item()) == 0, "device error flags %d" % int(out["error_flags"].item())
    gpu = parity.to_numpy(out, requests)
    lw = inp["log_weights"].cpu()
    gpu["log_weights"] = (lw if requests is None else lw[list(requests)]).numpy()
    rc_after = inp["refcount"].cpu().numpy() if pages else None
    ora = oracle.round(host, V=w.V, mode=w.mode, ess_frac=w.ess_frac, tv=w.tv, with_pages=pages)
    assert ora["status"] == 0
    stats = parity.check_round(host, ora, gpu, N=w.N, mode=w.mode, ess_frac=w.ess_frac,
                               tv=w.tv, pages=pages, rc_before=rc_before, rc_after=rc_after)
    _say("  ok", stats)
    return inp, out, ora, gpu


# ---------------------------------------------------------------- scaled-down workloads
SMALL = [
    W["r1-n8-k4-v32000-f32"].scaled(R=2),
    W["r16-n16-k4-v128256-bf16"].scaled(R=3, V=40000, ctx=256),
    W["r64-n32-k8-v128256-bf16-tv"].scaled(R=2, V=20000, ctx=256),
    W["r8-n16-k4-v152064-bf16-zipf-ess"].scaled(R=3, V=30000, ctx=1024),
    W["r32-n32-k8-v256000-bf16-tv-mixT"].scaled(R=4, V=36000, ctx=256),
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_scaled_workloads(w, dev):
    run_and_compare(w, dev, seed=1)


@pytest.mark.parametrize("V,dtype,tv", [(1, "bf16", True), (7, "f32", True), (8, "bf16", False),
                                        (9, "bf16", True), (33, "f32", False),
                                        (5001, "bf16", True), (16385, "bf16", True),
                                        (16384 * 3 + 8, "bf16", True), (8191, "f32", True),
                                        (524288, "bf16", True), (524281, "bf16", True), (262144, "f32", True),
                                        (1048576, "bf16", True), (1048569, "bf16", True), (524288, "f32", True)])
def test_ragged_and_tiny_vocabularies(V, dtype, tv, dev):
    w = W["r16-n16-k4-v128256-bf16"].scaled(name="ragged", R=2, N=8, K=3, V=V, dtype=dtype,
                                            tv=tv, ctx=128)
    run_and_compare(w, dev, seed=2, ragged=True)


@pytest.mark.parametrize("mode,tv", [("always", True), ("never", False), ("ess", True)])
def test_log_potential(mode, tv, dev):
    """Optional per-particle log potential (tilted target p*phi), with removed particles."""
    w = W["r64-n32-k8-v128256-bf16-tv"].scaled(name="potential", R=3, V=20000, ctx=128,
                                                mode=mode, tv=tv)

    def add(inp):
        inp["log_potential"] = synth.make_log_potential(w.R, w.N, 7, dev)

    inp, out, ora, gpu = run_and_compare(w, dev, seed=9, modify=add)
    removed = torch.isinf(inp["log_potential"]).cpu().numpy()
    assert removed.any()
    if mode == "always":
        dead = [set(np.nonzero(removed[r])[0]) for r in range(w.R)]
        assert all(not (set(gpu["ancestors"][r].tolist()) & dead[r]) for r in range(w.R))


@pytest.mark.parametrize("mode", ["never", "ess", "always"])
def test_potential_with_split_table(mode, dev):
    """A table of 32 x 256 entries a request, split by columns over four finalize workgroups
    a request, each redoing the weights from the previous log-weights (carried over in
    "never" and "ess"), with a log potential that removes particles."""
    w = W["r64-n32-k8-v128256-bf16-tv"].scaled(name="potential-split", R=3, V=20000, ctx=4096,
                                                mode=mode, ess_frac=0.7)
    assert w.N * w.P > 2048

    def add(inp):
        inp["log_potential"] = synth.make_log_potential(w.R, w.N, 11, dev)
        g = torch.Generator(device=dev)
        g.manual_seed(13)
        x = torch.randn(w.R, w.N, generator=g, device=dev)
        inp["log_weights"].copy_(torch.log_softmax(x, dim=1))   # unequal previous weights

    run_and_compare(w, dev, seed=12, modify=add)


@pytest.mark.parametrize("N,K", [(1, 1), (1, 4), (3, 1), (1024, 2), (40, 17), (2, 256)])
def test_particle_and_position_extremes(N, K, dev):
    w = W["r64-n32-k8-v128256-bf16-tv"].scaled(name="extreme", R=2, N=N, K=K, V=3000, ctx=64)
    run_and_compare(w, dev, seed=3)


@pytest.mark.parametrize("mode,frac", [("never", 0.5), ("ess", 0.5), ("ess", 1.0), ("always", 0.5)])
def test_resample_modes(mode, frac, dev):
    w = W["r8-n16-k4-v152064-bf16-zipf-ess"].scaled(name="modes", R=6, V=12000, ctx=256,
                                                    mode=mode, ess_frac=frac)
    run_and_compare(w, dev, seed=4)


def test_identical_target_and_draft(dev):
    w = W["r64-n32-k8-v128256-bf16-tv"].scaled(name="p-equals-q", R=3, V=20000, ctx=128)

    def same(inp):
        K = w.K
        inp["draft"].copy_(inp["target"][:, :, :K])
        inp["uniform"].copy_(torch.tensor([0.0, 0.5, 1.0 - 2.0 ** -24], device=dev))

    inp, out, ora, gpu = run_and_compare(w, dev, seed=5, modify=same)
    assert np.all(gpu["log_w_incr"] == 0.0)
    assert np.all(gpu["tv"] == 0.0)
    assert np.all(gpu["ess"] == w.N)
    assert np.all(gpu["ancestors"] == np.arange(w.N))


def test_extreme_logit_ranges(dev):
    # slices whose max lies hundreds of nats below the row max (their exponentials underflow
    # to 0) and rows whose draft is far from the target must give finite, exact-to-tolerance
    # weights and TV
    w = W["r64-n32-k8-v128256-bf16-tv"].scaled(name="extreme-range", R=2, N=4, K=3, V=40000,
                                               ctx=64)

    def widen(inp):
        inp["target"][:, :, :, 5000:30000] -= 300.0
        inp["draft"][:, 1:, :, 20000:39000] -= 250.0
        inp["target"][:, 0, 0, 7] += 200.0

    run_and_compare(w, dev, seed=10, modify=widen)


@pytest.mark.parametrize("tv", [True, False])
def test_all_negative_logits(tv, dev):
    # every logit below -20: each wave's share of each slice is negative, so its maximum comes
    # from the int16-min branch of the packed bf16 max (a constant shift leaves the softmax,
    # and so the drafted tokens, as they were)
    w = W["r64-n32-k8-v128256-bf16-tv"].scaled(name="all-negative", R=2, N=4, K=3, V=20000,
                                               ctx=64, tv=tv)

    def shift(inp):
        inp["target"].sub_(48.0)
        inp["draft"].sub_(48.0)
        assert float(inp["target"].float().max()) < 0 and float(inp["draft"].float().max()) < 0

    run_and_compare(w, dev, seed=11, modify=shift)


@pytest.mark.parametrize("tv", [True, False])
def test_masked_vocabulary_range(tv, dev):
    # the first half of every target and draft row is -inf (a masked range covering whole
    # slices): those slices add nothing, and nothing becomes NaN; drafted tokens lie in the
    # unmasked half
    w = W["r64-n32-k8-v128256-bf16-tv"].scaled(name="masked", R=2, N=4, K=3, V=40000, ctx=64,
                                               tv=tv)

    def mask(inp):
        inp["target"][..., : w.V // 2] = float("-inf")
        inp["draft"][..., : w.V // 2] = float("-inf")
        g = torch.Generator(device=dev)
        g.manual_seed(3)
        inp["tokens"].copy_(torch.randint(w.V // 2, w.V, inp["tokens"].shape, generator=g,
                                          device=dev, dtype=torch.int32))

    _, _, _, gpu = run_and_compare(w, dev, seed=12, modify=mask)
    assert np.all(np.isfinite(gpu["log_w_incr"])) and np.all(gpu["bonus"] >= w.V // 2)


@pytest.mark.parametrize("tv", [True, False])
def test_row_max_at_every_chunk_position(tv, dev):
    # a +200 spike (its exp overflows unless the slice max sees it) at each of the 8 element
    # positions of a 16-byte chunk, in different rows, plus one at the row's last element
    w = W["r64-n32-k8-v128256-bf16-tv"].scaled(name="spikes", R=1, N=10, K=2, V=20001, ctx=64,
                                               tv=tv)

    def spike(inp):
        for i in range(8):
            inp["target"][0, i, 0, 8 * 37 + i] += 200.0
            inp["draft"][0, i, 1, 8 * 1000 + i] += 200.0
        inp["target"][0, 8, 1, w.V - 1] += 200.0
        inp["draft"][0, 9, 0, w.V - 1] += 200.0

    run_and_compare(w, dev, seed=11, modify=spike)


def test_empty_batch(dev):
    w = W["r16-n16-k4-v128256-bf16"].scaled(name="empty", R=0, V=1000, ctx=64)
    inp = synth.make_inputs(w, 0, device=dev, pages=False)
    out = smcsd.run_round(inp, pages=False)
    torch.cuda.synchronize()
    assert out["ancestors"].numel() == 0


# ---------------------------------------------------------------- full-size workloads
@pytest.mark.parametrize("name", ["r1-n8-k4-v32000-f32", "r16-n16-k4-v128256-bf16",
                                  "r8-n16-k4-v152064-bf16-zipf-ess"])
def test_full_size_workloads(name, dev):
    run_and_compare(W[name], dev, seed=0)


@pytest.mark.parametrize("name", ["r64-n32-k8-v128256-bf16-tv", "r32-n32-k8-v256000-bf16-tv-mixT"])
def test_full_size_tv_workloads(name, dev):
    """Every request of the two TV workloads at full size, in the launch configuration the
    benchmark times (persistent grid over all row pairs, every temperature switch)."""
    _, _, ora, gpu = run_and_compare(W[name], dev, seed=0)
    assert gpu["tv"].min() >= 0 and gpu["tv"].max() <= 1


# ---------------------------------------------------------------- determinism
def test_bitwise_deterministic(dev):
    w = W["r64-n32-k8-v128256-bf16-tv"].scaled(name="determinism", R=8, V=40000, ctx=256)
    inp = synth.make_inputs(w, 6, device=dev)
    lw0 = inp["log_weights"].clone()
    rc0 = inp["refcount"].clone()
    outs = []
    for _ in range(2):
        inp["log_weights"].copy_(lw0)
        inp["refcount"].copy_(rc0)
        o = smcsd.run_round(inp, tv=True)
        torch.cuda.synchronize()
        outs.append({k: v.clone() for k, v in o.items() if k != "workspace" and v is not None})
        outs[-1]["log_weights"] = inp["log_weights"].clone()
        outs[-1]["refcount"] = inp["refcount"].clone()
    for k in outs[0]:
        assert torch.equal(outs[0][k], outs[1][k]), k


# ---------------------------------------------------------------- multi-round state
def test_three_rounds_with_carried_state(dev):
    w = W["r16-n16-k4-v128256-bf16"].scaled(name="three-rounds", R=4, V=9000, ctx=256,
                                            tv=True)
    inp = synth.make_inputs(w, 7, device=dev)
    for t in range(3):
        _say("round", t)
        inp2 = synth.make_inputs(w, 100 + t, device=dev, pages=False)   # fresh logits
        for k in ("target", "draft", "tokens", "gumbel", "uniform"):
            inp[k] = inp2[k]
        _, out, _, _ = run_and_compare(w, dev, inputs=inp)
        # pointer exchange between rounds: the output table becomes the next input
        inp["page_table"], out["page_table_out"] = out["page_table_out"], inp["page_table"]


# ---------------------------------------------------------------- standalone entry points
@pytest.mark.parametrize("N,mode", [(1, "always"), (7, "always"), (32, "ess"), (1000, "always"),
                                    (64, "never")])
def test_smcsd_resample(N, mode, dev):
    R = 5
    g = torch.Generator().manual_seed(N)
    lw = (torch.randn(R, N, generator=g) * 2).float()
    prev = torch.log_softmax(torch.randn(R, N, generator=g).double(), 1).float()
    u = torch.rand(R, generator=g).float()
    d = dict(log_w_incr=lw.to(dev), log_weights=prev.to(dev), uniform=u.to(dev),
             log_norm=torch.empty(R, device=dev), ess=torch.empty(R, device=dev),
             resampled=torch.empty(R, dtype=torch.int32, device=dev),
             ancestors=torch.empty(R, N, dtype=torch.int32, device=dev))
    smcsd.smcsd_resample(**d, mode=mode, ess_frac=0.5)
    torch.cuda.synchronize()
    for r in range(R):
        ref = oracle.resample_request(lw[r].double().numpy(), prev[r].double().numpy(),
                                      float(u[r]), mode, 0.5)
        assert int(d["resampled"][r]) == ref["resampled"]
        assert float(d["log_norm"][r]) == pytest.approx(ref["log_norm"], rel=1e-6, abs=1e-6)
        assert float(d["ess"][r]) == pytest.approx(ref["ess"], rel=1e-6)
        safe = ref["anc_gap"] >= 1e-9
        assert np.array_equal(d["ancestors"][r].cpu().numpy()[safe], ref["ancestors"][safe])
        np.testing.assert_allclose(d["log_weights"][r].cpu().numpy(), ref["log_weights"],
                                   rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("frac,resampled", [(0.25, 0), (0.25 + 2.0 ** -20, 1)])
def test_smcsd_resample_ess_exactly_at_threshold(frac, resampled, dev):
    """N = 8, two particles at log weight 0 and six at -1e4: W = (1/2, 1/2, 0, ...) exactly and
    ESS = 2 exactly. With ess_frac = 0.25 the threshold is 2 and the strict ESS < 2 keeps the
    weights; a threshold a hair above 2 resamples (each survivor duplicated 4 times)."""
    R, N = 3, 8
    lw = torch.full((R, N), -1e4)
    lw[:, 2] = 0.0
    lw[:, 5] = 0.0
    prev = torch.full((R, N), -math.log(N))
    u = torch.tensor([0.0, 0.3, 0.999])
    d = dict(log_w_incr=lw.to(dev), log_weights=prev.clone().to(dev), uniform=u.to(dev),
             log_norm=torch.empty(R, device=dev), ess=torch.empty(R, device=dev),
             resampled=torch.empty(R, dtype=torch.int32, device=dev),
             ancestors=torch.empty(R, N, dtype=torch.int32, device=dev))
    smcsd.smcsd_resample(**d, mode="ess", ess_frac=frac)
    torch.cuda.synchronize()
    assert torch.all(d["ess"].cpu() == 2.0)
    assert torch.all(d["resampled"].cpu() == resampled)
    for r in range(R):
        ref = oracle.resample_request(lw[r].double().numpy(), prev[r].double().numpy(),
                                      float(u[r]), "ess", frac)
        assert ref["ess"] == 2.0 and ref["resampled"] == resampled
        assert np.array_equal(d["ancestors"][r].cpu().numpy(), ref["ancestors"])
        np.testing.assert_allclose(d["log_weights"][r].cpu().numpy(), ref["log_weights"],
                                   rtol=1e-6, atol=1e-6)
    if resampled:
        assert np.array_equal(d["ancestors"][0].cpu().numpy(), [2] * 4 + [5] * 4)


@pytest.mark.parametrize("N,ctx", [(16, 1024), (128, 1024), (32, 3200), (128, 4096), (100, 1600),
                                   (16, 9600), (8, 16384), (1, 131072), (24, 14000), (64, 2608),
                                   (8, 65536), (1, 262144)])
def test_round_remap_with_repeated_pages(N, ctx, dev):
    # Page ids repeated across rows in any order and across columns, some columns one page for
    # every row. The round's remap (one atomic per run of equal pages in a column up to 64
    # particles, one per entry above) must still give every page the sum over its entries.
    # Up to 64 particles the small finalize kernel remaps the table from LDS, in one workgroup
    # a request up to 2048 entries (N * P = 1024), else split by columns over several
    # workgroups a request: 6400 entries over 4 of 50 columns, 9600 over 5 of 120, 8192 over
    # 4 of 256, N = 1 and P = 8192 over 4 of 2048, 21000 over 11 of 79-80, 10432 over 6 of
    # 27-28, 32768 over 16 of 256, N = 1 and P = 16384 over 8. Above 64 particles the general
    # finalize kernel remaps up to 8192 entries (128 particles) and the remap kernel larger
    # ones over several workgroups (10000 by rows with a stride that is no multiple of
    # P = 100, 32768).
    w = W["r64-n32-k8-v128256-bf16-tv"].scaled(name="repeated-pages", R=3, N=N, K=2, V=3000,
                                               ctx=ctx)

    def tables(inp):
        R, n, P = inp["page_table"].shape
        g = torch.Generator().manual_seed(12)
        pool = 40
        pt = torch.randint(0, pool, (R, n, P), generator=g, dtype=torch.int32)
        pt[:, :, :4] = pt[:, :1, :4]                                   # kept by every row
        pt[torch.rand(R, n, P, generator=g) < 0.1] = -1                # unused entries
        pt = torch.where(pt >= 0, pt + pool * torch.arange(R, dtype=torch.int32).view(R, 1, 1), pt)
        rc = torch.bincount(pt[pt >= 0].long(), minlength=R * pool).to(torch.int32)
        inp["page_table"] = pt.to(dev).contiguous()
        inp["refcount"] = rc.to(dev).contiguous()

    run_and_compare(w, dev, seed=12, modify=tables)


def test_smcsd_remap_pages_and_error_flags(dev):
    R, N, P = 3, 16, 40
    pt, rc, npg = synth.make_page_table(R, N, P, seed=8, ragged=True)
    g = torch.Generator().manual_seed(8)
    anc = torch.sort(torch.randint(0, N, (R, N), generator=g), 1).values.int()
    pt_out = torch.empty_like(pt, device=dev)
    rc_d = rc.to(dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    smcsd.smcsd_remap_pages(ancestors=anc.to(dev), page_table_in=pt.to(dev),
                            page_table_out=pt_out, refcount=rc_d, error_flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    rc_ref = rc.numpy().copy()
    for r in range(R):
        out_r, rc_ref, st = oracle.remap_request(anc[r].numpy(), pt[r].numpy(), rc_ref)
        assert st == 0
        assert np.array_equal(pt_out[r].cpu().numpy(), out_r)
    assert np.array_equal(rc_d.cpu().numpy(), rc_ref)
    # an out-of-range ancestor and page id are flagged and skipped, never followed
    bad_anc = anc.clone()
    bad_anc[1, 3] = N + 5
    bad_pt = pt.clone()
    bad_pt[2, 0, 0] = npg + 100
    flags.zero_()
    smcsd.smcsd_remap_pages(ancestors=bad_anc.to(dev), page_table_in=bad_pt.to(dev),
                            page_table_out=pt_out, refcount=rc.to(dev).clone(), error_flags=flags)
    torch.cuda.synchronize()
    f = int(flags.item())
    assert f & smcsd.DEVERR_ANCESTOR
    assert torch.all(pt_out[1, 3] == -1)


def test_out_of_range_token_is_flagged(dev):
    w = W["r16-n16-k4-v128256-bf16"].scaled(name="bad-token", R=2, V=3000, ctx=64)
    inp = synth.make_inputs(w, 9, device=dev)
    inp["tokens"][1, 2, 0] = w.V + 7
    out = smcsd.run_round(inp)
    torch.cuda.synchronize()
    assert int(out["error_flags"].item()) & smcsd.DEVERR_TOKEN
    assert torch.isfinite(out["log_w_incr"]).all()


# ---------------------------------------------------------------- failure handling
def test_exchange_time_limit_aborts_and_drains(dev, monkeypatch):
    """A wait limit of 0 ticks, set from the host, makes every exchange that is not complete
    at its first poll time out. The workgroup that times out raises the abort flag and
    SMCSD_DEVERR_EXCHANGE, every later wait returns at once, and the kernel drains. The next
    call, with the normal limit, is correct again on the same workspace."""
    w = W["r64-n32-k8-v128256-bf16-tv"].scaled(name="abort", R=2, N=8, K=4, ctx=256)
    inp = synth.make_inputs(w, 4, device=dev)
    out = smcsd.alloc_outputs(w.R, w.N, w.K, dev, tv=True, V=w.V)
    monkeypatch.setenv("SMCSD_EXCHANGE_TIMEOUT_TICKS", "0")
    _say("case abort: time limit 0")
    smcsd.run_round({k: (v.clone() if torch.is_tensor(v) else v) for k, v in inp.items()},
                    mode=w.mode, tv=True, outputs=out)
    torch.cuda.synchronize()
    flags = int(out["error_flags"].item())
    assert flags & smcsd.DEVERR_EXCHANGE, flags
    monkeypatch.delenv("SMCSD_EXCHANGE_TIMEOUT_TICKS")
    out["error_flags"].zero_()
    out["page_table_out"] = torch.empty_like(inp["page_table"])
    _say("case abort: normal limit on the same workspace")
    host = synth.to_host(inp)
    rc_before = inp["refcount"].cpu().numpy().copy()
    smcsd.run_round(inp, mode=w.mode, tv=True, outputs=out)
    torch.cuda.synchronize()
    assert int(out["error_flags"].item()) == 0
    gpu = parity.to_numpy(out)
    gpu["log_weights"] = inp["log_weights"].cpu().numpy()
    ora = oracle.round(host, V=w.V, mode=w.mode, tv=True)
    parity.check_round(host, ora, gpu, N=w.N, mode=w.mode, tv=True, rc_before=rc_before,
                       rc_after=inp["refcount"].cpu().numpy())
