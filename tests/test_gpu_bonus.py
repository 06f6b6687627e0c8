"""GPU parity of the bonus token drawn after resampling (smcsd_bonus_resampled, through the
C ABI) against the oracle, and of the round run without in-pass noise.

The SMC-SD page (section 2) yields K + 1 tokens per particle and round without fixing when
the last one is drawn; this reading draws it per new slot from the ancestor's bonus row with
the slot's own noise row, by the Gumbel-max key of the STAND page (method item 2, k = 1).
Tokens are compared bit for bit wherever the oracle's top-2 gap of the exact key z/T + G is
>= 1e-5; in a nearer tie the GPU's token must be a valid winner (tests/parity.py).
"""
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


def _host(t):
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _bonus_gpu(inp, anc, noise, dev, out_tokens=None):
    R, N, K1, ld = inp["target"].shape
    dt = smcsd.BF16 if inp["target"].dtype == torch.bfloat16 else smcsd.F32
    ws = torch.empty(max(256, smcsd.smcsd_bonus_workspace_size(R, N, inp["V"], dt)),
                     dtype=torch.uint8, device=dev)
    bonus = torch.full((R, N), -9, dtype=torch.int32, device=dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    smcsd.smcsd_bonus_resampled(target_logits=inp["target"], temperature=inp["temperature"],
                                ancestors=anc, gumbel=noise, bonus=bonus, workspace=ws,
                                out_tokens=out_tokens, error_flags=flags, V=inp["V"])
    torch.cuda.synchronize()
    return bonus.cpu().numpy(), int(flags.item())


CASES = [
    W["r1-n8-k4-v32000-f32"].scaled(R=2),
    W["r16-n16-k4-v128256-bf16"].scaled(R=3, V=40001),           # ragged last chunk
    W["r64-n32-k8-v128256-bf16-tv"].scaled(R=4),                 # full vocabulary
    W["r64-n32-k8-v128256-bf16-tv"],                             # the headline shape
    W["r32-n32-k8-v256000-bf16-tv-mixT"].scaled(R=3, V=70000),   # mixed temperatures
    W["r16-n16-k4-v128256-bf16"].scaled(R=2, N=1024, K=1, V=3000),
    W["r1-n8-k4-v32000-f32"].scaled(R=3, N=5, K=2, V=1),
]


@pytest.mark.parametrize("w", CASES, ids=["%s-R%d-N%d-K%d-V%d" % (w.name, w.R, w.N, w.K, w.V)
                                          for w in CASES])
def test_bonus_resampled_matches_oracle(w, dev):
    _say("case", w.name, "R N K V", w.R, w.N, w.K, w.V)
    inp = synth.make_inputs(w, 5, device=dev, pages=False)
    noise = synth.make_gumbel(w, 6, device=dev)
    anc = synth.make_ancestors(w.R, w.N, 7, device=dev)
    out_tok = torch.full((w.R, w.N, w.K + 1), -5, dtype=torch.int32, device=dev)
    g, flags = _bonus_gpu(inp, anc, noise, dev, out_tokens=out_tok)
    assert flags == 0
    o = oracle.bonus_resampled(_host(inp["target"]), _host(inp["temperature"]), _host(anc),
                               _host(noise), V=w.V)
    assert o["status"] == 0
    h = _host(inp["target"])
    rows = h[np.arange(w.R)[:, None], _host(anc), w.K]              # ancestor's bonus row
    st = parity.check_bonus("bonus", g, o["bonus"], o["gap"], rows, _host(noise),
                            np.broadcast_to(_host(inp["temperature"])[:, None], g.shape), w.V)
    _say("  bonus", st)
    ot = out_tok.cpu().numpy()
    assert np.array_equal(ot[:, :, w.K], g) and (ot[:, :, :w.K] == -5).all()
    _say("  ok")


def test_out_of_range_ancestor_is_flagged(dev):
    w = W["r1-n8-k4-v32000-f32"].scaled(R=2, V=5000)
    inp = synth.make_inputs(w, 5, device=dev, pages=False)
    anc = synth.make_ancestors(w.R, w.N, 7, device=dev)
    anc[1, 3] = w.N
    anc[0, 0] = -1
    g, flags = _bonus_gpu(inp, anc, inp["gumbel"], dev)
    assert flags == smcsd.DEVERR_ANCESTOR
    o = oracle.bonus_resampled(_host(inp["target"]), _host(inp["temperature"]), _host(anc),
                               _host(inp["gumbel"]), V=w.V)
    assert o["status"] == -1 and g[1, 3] == -1 and g[0, 0] == -1
    ok = (anc.cpu().numpy() >= 0) & (anc.cpu().numpy() < w.N)
    h = _host(inp["target"])
    a = np.clip(_host(anc), 0, w.N - 1)
    rows = h[np.arange(w.R)[:, None], a, w.K]
    T = np.broadcast_to(_host(inp["temperature"])[:, None], g.shape)
    parity.check_bonus("bonus", g[ok], o["bonus"][ok], o["gap"][ok], rows[ok],
                       _host(inp["gumbel"])[ok], T[ok], w.V)


@pytest.mark.parametrize("tv", [False, True])
def test_round_without_noise_changes_only_the_bonus(tv, dev):
    """gumbel = NULL: the same weights, ancestors, tables and TV as the full round, no bonus
    written, column K of out_tokens -1."""
    w = W["r16-n16-k4-v128256-bf16"].scaled(R=3, V=30000, ctx=256, tv=tv)
    base = synth.make_inputs(w, 8, device=dev)
    outs = []
    for noise in (True, False):
        inp = {k: (v.clone() if torch.is_tensor(v) else v) for k, v in base.items()}
        if not noise:
            inp["gumbel"] = None
        out = smcsd.alloc_outputs(w.R, w.N, w.K, dev, tv=tv, V=w.V)
        out["bonus"].fill_(-7)
        pt_out = torch.empty_like(inp["page_table"])
        smcsd.smcsd_round(target_logits=inp["target"], draft_logits=inp["draft"],
                          draft_tokens=inp["tokens"], temperature=inp["temperature"],
                          gumbel=inp["gumbel"], uniform=inp["uniform"],
                          log_weights=inp["log_weights"], log_w_incr=out["log_w_incr"],
                          log_norm=out["log_norm"], ess=out["ess"], resampled=out["resampled"],
                          ancestors=out["ancestors"], bonus=out["bonus"],
                          out_tokens=out["out_tokens"], tv=out["tv"],
                          page_table_in=inp["page_table"], page_table_out=pt_out,
                          refcount=inp["refcount"], error_flags=out["error_flags"],
                          workspace=out["workspace"], V=w.V)
        torch.cuda.synchronize()
        assert int(out["error_flags"].item()) == 0
        out.update(page_table_out=pt_out, log_weights=inp["log_weights"], refcount=inp["refcount"])
        outs.append(out)
    full, bare = outs
    for k in ("log_w_incr", "log_norm", "ess", "resampled", "ancestors", "log_weights",
              "page_table_out", "refcount") + (("tv",) if tv else ()):
        assert torch.equal(full[k], bare[k]), k
    assert (bare["bonus"] == -7).all()
    assert torch.equal(full["out_tokens"][:, :, :w.K], bare["out_tokens"][:, :, :w.K])
    assert (bare["out_tokens"][:, :, w.K] == -1).all()


@pytest.mark.parametrize("mode", ["always", "ess"])
def test_round_then_bonus_after_resampling(mode, dev):
    """run_round(bonus_noise=...) against the oracle's round and its bonus_resampled on the
    oracle's own ancestors."""
    w = W["r64-n32-k8-v128256-bf16-tv"].scaled(R=3, V=20000, ctx=256, mode=mode)
    inp = synth.make_inputs(w, 9, device=dev)
    noise = synth.make_gumbel(w, 10, device=dev)
    host = synth.to_host(inp)
    out = smcsd.run_round(inp, mode=mode, ess_frac=w.ess_frac, tv=w.tv, bonus_noise=noise)
    torch.cuda.synchronize()
    assert int(out["error_flags"].item()) == 0
    ora = oracle.round(host, V=w.V, mode=mode, ess_frac=w.ess_frac, tv=w.tv)
    assert np.all(ora["anc_gap"] >= parity.ANC_GAP), "near tie: pick another seed"
    if mode == "ess":
        assert np.all(np.abs(ora["ess"] - w.ess_frac * w.N) >= 1e-4 * w.N), "ESS at threshold"
    anc = out["ancestors"].cpu().numpy()
    assert np.array_equal(anc, ora["ancestors"])
    ob = oracle.bonus_resampled(host["target"], host["temperature"], ora["ancestors"],
                                _host(noise), V=w.V)
    gb = out["bonus"].cpu().numpy()
    rows = host["target"][np.arange(w.R)[:, None], anc, w.K]
    parity.check_bonus("bonus", gb, ob["bonus"], ob["gap"], rows, _host(noise),
                       np.broadcast_to(host["temperature"][:, None], gb.shape), w.V)
    drafted = host["tokens"][np.arange(w.R)[:, None], anc]          # [R, N, K]
    want = np.concatenate([drafted, gb[:, :, None]], axis=2)
    assert np.array_equal(out["out_tokens"].cpu().numpy(), want)
