"""GPU parity of Gumbel-Top-K (smcsd_gumbel_topk) against the oracle, through the C ABI.

The oracle ranks the exact keys z/T + G (in double); the GPU ranks binary32 keys
fl32(fma(z, fl32(1/T), G)), whose error is at most 2^-24 (|z/T| + |key|) each. The bar:
  * a rank whose oracle gaps to both neighbouring ranks are >= 1e-5 has one correct token,
    and the GPU's must be it (bit-exact);
  * every rank: the GPU's tokens are distinct and in range, the exact key of the GPU's token
    lies within 1e-5 of the oracle's key at that rank, the GPU's keys do not increase, and
    each GPU key lies within the binary32 bound above of its token's exact key.
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


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _host(t):
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def compare(logits, temp, noise, k, V, rows_checked=None):
    _say("topk case rows", logits.shape[0], "ld", logits.shape[1], "V", V, "k", k, logits.dtype)
    out = smcsd.gumbel_topk(logits, temp, noise, k, V=V)
    torch.cuda.synchronize()
    tok, key = out["tokens"].cpu().numpy(), out["keys"].cpu().numpy()
    sel = slice(None) if rows_checked is None else rows_checked
    z, T, G = _host(logits[sel]), _host(temp[sel]), _host(noise[sel])
    tok_s, key_s = tok[sel], key[sel].astype(np.float64)
    otok, okey, ogap = oracle.gumbel_topk(z, T, G, k, V=V, gaps=True)
    rows = otok.shape[0]
    assert np.all((tok_s >= 0) & (tok_s < V))
    assert all(len(set(r.tolist())) == k for r in tok_s)
    before = np.concatenate([np.full((rows, 1), np.inf), ogap[:, :-1]], 1)
    unique = (ogap >= parity.KEY_GAP) & (before >= parity.KEY_GAP)
    bad = unique & (tok_s != otok)
    assert not bad.any(), ("tokens", np.argwhere(bad)[:5].tolist())
    kg = parity.exact_keys(z, G, np.asarray(T), tok_s)
    assert np.all(np.abs(kg - okey) <= parity.KEY_GAP), np.argwhere(np.abs(kg - okey) > parity.KEY_GAP)[:5]
    assert np.all(np.diff(key_s, axis=1) <= 0)
    zT = kg - np.take_along_axis(np.asarray(G, np.float64), tok_s, 1)
    bound = 2.0 ** -24 * (np.abs(zT) + np.abs(kg)) * (1 + 1e-6)
    assert np.all(np.abs(key_s - kg) <= bound), np.argwhere(np.abs(key_s - kg) > bound)[:5]
    _say("  ok: ranks compared %d, near ties %d" % (int(unique.sum()), int((~unique).sum())))
    return tok, key, otok


@pytest.mark.parametrize("k", [1, 2, 8, 17, 64])
def test_topk_k_values(k, dev):
    w = W["r64-n32-k8-v128256-bf16-tv"].scaled(name="topk", R=2, N=8, V=40000, ctx=64)
    inp = synth.make_inputs(w, 1, device=dev, pages=False)
    z, T, G = synth.topk_rows(inp)
    compare(z, T, G, k, w.V)


@pytest.mark.parametrize("V,dtype,k", [(1, "bf16", 1), (9, "bf16", 9), (7, "f32", 3),
                                       (64, "bf16", 64), (5001, "bf16", 13), (16385, "f32", 8),
                                       (1048569, "bf16", 8), (524288, "f32", 5),
                                       (1048569, "bf16", 64), (300000, "f32", 40),
                                       (933888, "bf16", 9)])
def test_topk_ragged_and_maximal(V, dtype, k, dev):
    # V = 1048569 bf16 is 64 slices: k = 8 gives 512 candidates a row (the most the one-wave
    # merge takes), k = 64 the most of all (4096); 300000 f32 is 37 slices, k = 40 1480;
    # 933888 bf16 is 57 slices, k = 9 513 (one past the one-wave merge)
    w = W["r16-n16-k4-v128256-bf16"].scaled(name="topk-ragged", R=2, N=3, V=V, dtype=dtype, ctx=64)
    inp = synth.make_inputs(w, 2, device=dev, pages=False)
    z, T, G = synth.topk_rows(inp)
    compare(z, T, G, k, V)


def test_topk_heavy_ties(dev):
    """Zero noise and logits taking only a few values: ranking is decided by index."""
    rows, V, k = 6, 30000, 40
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    z = torch.randint(0, 4, (rows, V), generator=g, device=dev).to(torch.bfloat16)
    T = torch.ones(rows, dtype=torch.float32, device=dev)
    G = torch.zeros((rows, V), dtype=torch.float32, device=dev)
    tok, _, otok = compare(z, T, G, k, V)
    assert np.all(np.diff(tok, axis=1) > 0)      # all keys equal -> increasing indices
    # z in {0..3}, T = 1, G = 0: every binary32 key is exact, so the GPU decides exactly as
    # the oracle, ties included
    assert np.array_equal(tok, otok)


def test_topk_full_size_sampled(dev):
    """2048 rows of V = 128256 bf16 (the headline shape's particles), k = 8; the oracle checks
    a sample of rows."""
    w = W["r64-n32-k8-v128256-bf16-tv"]
    inp = synth.make_inputs(w, 4, device=dev, pages=False)
    z, T, G = synth.topk_rows(inp)
    compare(z, T, G, 8, w.V, rows_checked=[0, 1, 777, 2047])
