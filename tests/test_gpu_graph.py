"""The library's launch sequences under HIP graph capture.

Every entry point enqueues kernels only: no memset node, no allocation, no host
synchronisation. So a caller can capture a round, or a whole driver step (round + page
lifecycle), into a graph and replay it. Each replay here starts from the same restored state,
with eager work and synchronisations between replays, and must reproduce the eager results
bit for bit (the kernels are deterministic).
"""
import pytest
import torch

from smc_particle_resampling_amd import smcsd, synth

pytestmark = pytest.mark.gpu
W = synth.WORKLOADS


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


@pytest.mark.parametrize("tv", [False, True])
def test_driver_step_replays_in_a_graph(tv, dev):
    w = W["r16-n16-k4-v128256-bf16"].scaled(R=3, V=30000, ctx=256, tv=tv, mode="ess")
    K, ps, P = w.K, 16, 12
    inp = synth.make_inputs(w, 3, device=dev, pages=False)
    pool = synth.make_page_pool(w.R, w.N, P, ps, 4, steps=K + 1, spare=300, kv_count=2,
                                page_bytes=64)
    state0 = dict(log_weights=inp["log_weights"].clone(), page_table=pool["page_table"].to(dev),
                  refcount=pool["refcount"].to(dev), free_ids=pool["free_ids"].to(dev),
                  n_free=torch.tensor([pool["n_free"]], dtype=torch.int32, device=dev),
                  kv=pool["kv"].to(dev))
    st = {k: v.clone() for k, v in state0.items()}
    inp.update(log_weights=st["log_weights"], page_table=st["page_table"], refcount=st["refcount"])
    lb, la = pool["len_before"].to(dev), pool["len_after"].to(dev)
    out = smcsd.alloc_outputs(w.R, w.N, w.K, dev, tv=tv, V=w.V)
    out["page_table_out"] = torch.empty_like(st["page_table"])
    pws = torch.empty(smcsd.smcsd_pages_workspace_size(w.R, w.N, P, st["refcount"].numel()),
                      dtype=torch.uint8, device=dev)
    stats = torch.zeros(5, dtype=torch.int32, device=dev)

    def step():
        smcsd.run_round(inp, mode=w.mode, ess_frac=w.ess_frac, tv=tv, outputs=out)
        smcsd.smcsd_pages_advance(len_before=lb, len_after=la, page_table=out["page_table_out"],
                                  refcount=st["refcount"], free_ids=st["free_ids"],
                                  n_free=st["n_free"], page_size=ps, workspace=pws,
                                  kv=st["kv"], stats=stats, error_flags=out["error_flags"])

    def restore():
        for k, v in state0.items():
            st[k].copy_(v)
        out["error_flags"].zero_()

    def snapshot():
        keys = ["log_w_incr", "log_norm", "ess", "resampled", "ancestors", "bonus", "out_tokens",
                "page_table_out", "error_flags"] + (["tv"] if tv else [])
        snap = {k: out[k].clone() for k in keys}
        snap.update({"state_" + k: v.clone() for k, v in st.items()}, stats=stats.clone())
        return snap

    step()
    torch.cuda.synchronize()
    assert int(out["error_flags"].item()) == 0
    ref = snapshot()
    assert int(ref["stats"][1]) > 0                       # the lifecycle did pop pages

    restore()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        restore()
        for k in ("ancestors", "bonus", "out_tokens", "page_table_out"):
            out[k].fill_(-3)
        stats.fill_(-3)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for k in ref:
            assert torch.equal(got[k], ref[k]), (rep, k)
        torch.randn(4096, device=dev).sum().item()        # eager work between replays
