"""GPU test of smcsd_round_noalloc (through the C ABI): the round with the library's static
scratch buffer as its workspace must give exactly what smcsd_round gives with a workspace of
the caller's, on the same inputs. Two calls in a row, the second on a smaller input, so the
second finds the first's contents in the buffer."""
import sys

import pytest
import torch

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


def _round(inp, noalloc, dev, tv, mode):
    """One round on a private copy of the in/out state; returns every output."""
    w_in = {k: (v.clone() if torch.is_tensor(v) else v) for k, v in inp.items()}
    R, N, K1, ld = w_in["target"].shape
    K = K1 - 1
    out = smcsd.alloc_outputs(R, N, K, dev, tv=tv, V=w_in["V"])
    out["page_table_out"] = torch.full_like(w_in["page_table"], -7)
    kw = dict(target_logits=w_in["target"], draft_logits=w_in["draft"],
              draft_tokens=w_in["tokens"], temperature=w_in["temperature"],
              gumbel=w_in["gumbel"], uniform=w_in["uniform"], log_weights=w_in["log_weights"],
              log_w_incr=out["log_w_incr"], log_norm=out["log_norm"], ess=out["ess"],
              resampled=out["resampled"], ancestors=out["ancestors"], bonus=out["bonus"],
              out_tokens=out["out_tokens"], tv=out.get("tv"), page_table_in=w_in["page_table"],
              page_table_out=out["page_table_out"], refcount=w_in["refcount"],
              error_flags=out["error_flags"], V=w_in["V"], mode=mode, ess_frac=0.5)
    if noalloc:
        smcsd.smcsd_round_noalloc(**kw)
    else:
        smcsd.smcsd_round(workspace=out["workspace"], **kw)
    torch.cuda.synchronize()
    res = {k: v for k, v in out.items() if torch.is_tensor(v) and k != "workspace"}
    res["log_weights"] = w_in["log_weights"]
    res["refcount"] = w_in["refcount"]
    return res


CASES = [
    # the first call is the larger one: the headline shape with 8 requests, TV on
    (W["r64-n32-k8-v128256-bf16-tv"].scaled(name="noalloc-large", R=8), True, "always"),
    # then a smaller input: fewer requests and particles, a ragged V, TV on
    (W["r32-n32-k8-v256000-bf16-tv-mixT"].scaled(name="noalloc-small", R=2, N=8, K=3, V=20001,
                                                 ctx=128), True, "always"),
    # and without TV, ESS mode (different workspace layout, no exchange)
    (W["r8-n16-k4-v152064-bf16-zipf-ess"].scaled(name="noalloc-ess", R=3, V=30000, ctx=256,
                                                 tv=False), False, "ess"),
]


def test_noalloc_matches_round_twice_in_a_row(dev):
    for i, (w, tv, mode) in enumerate(CASES):
        _say("noalloc call", i, w.name, "R N K V", w.R, w.N, w.K, w.V, "tv", tv, "mode", mode)
        inp = synth.make_inputs(w, 20 + i, device=dev)
        ref = _round(inp, False, dev, tv, mode)
        got = _round(inp, True, dev, tv, mode)
        assert int(ref["error_flags"].item()) == 0 and int(got["error_flags"].item()) == 0
        for k in ref:
            assert torch.equal(ref[k], got[k]), (w.name, k)
        _say("  equal:", sorted(ref))
