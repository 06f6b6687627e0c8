"""CPU checks of the host-side tools: bench.py's contract pieces that need no GPU, and the
seeded generators of the page lifecycle's inputs (consistency of the pools they draw)."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import bench
from smc_particle_resampling_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2 and "one GPU" in p.stderr


def test_stored_traffic_needs_the_same_kernel_sources(monkeypatch):
    wl = synth.HEADLINE
    path = os.path.join(bench.PROFILES, "traffic_k_logits_%s.json" % wl)
    if not os.path.exists(path):
        pytest.skip("no traffic record")
    monkeypatch.setattr(bench, "kernel_source_hash", lambda kernel: "0000000000000000")
    assert bench.stored_traffic(wl, "k_logits_tv") is None


def test_kernel_source_hash_is_stable():
    for k in bench.KERNEL_SOURCES:
        assert bench.kernel_source_hash(k) == bench.kernel_source_hash(k)
        assert len(bench.kernel_source_hash(k)) == 16
    assert bench.kernel_source_hash("k_logits_tv") != bench.kernel_source_hash("k_logits_stream")


@pytest.mark.parametrize("R,N,P,ps,steps,spare", [(3, 8, 6, 4, None, 40), (4, 64, 20, 8, 8, 0),
                                                  (2, 1, 5, 16, 17, 5)])
def test_page_pool_is_consistent(R, N, P, ps, steps, spare):
    pool = synth.make_page_pool(R, N, P, ps, 9, steps=steps, spare=spare, kv_count=2,
                                page_bytes=32)
    pt = pool["page_table"].numpy()
    rc = pool["refcount"].numpy()
    num_pages = rc.size
    used = pt[pt >= 0]
    counts = np.bincount(used, minlength=num_pages)
    live = rc >= 0
    assert np.array_equal(rc[live], counts[live])            # refcount = entries naming it
    assert np.all(counts[~live] == 0)
    free = pool["free_ids"].numpy()[:pool["n_free"]]
    assert len(set(free.tolist())) == free.size == int((rc == -1).sum())
    assert np.all(rc[free] == -1)
    lb, la = pool["len_before"].numpy(), pool["len_after"].numpy()
    assert np.all(lb >= 1) and np.all(la >= lb) and np.all(la <= P * ps)
    cols = -(-lb // ps)
    for r in range(R):                                       # columns filled up to the length
        assert np.all(pt[r, :, :cols[r]] >= 0) and np.all(pt[r, :, cols[r]:] == -1)
    assert pool["kv"].shape == (2, num_pages, 32) and pool["kv"].dtype == torch.uint8
    # page ids of different requests are disjoint
    sets = [set(pt[r][pt[r] >= 0].tolist()) for r in range(R)]
    assert all(not (sets[a] & sets[b]) for a in range(R) for b in range(a + 1, R))


def test_ancestors_and_fresh_noise():
    anc = synth.make_ancestors(5, 16, 3).numpy()
    assert anc.shape == (5, 16) and anc.min() >= 0 and anc.max() < 16
    assert np.all(np.diff(anc, axis=1) >= 0)
    w = synth.WORKLOADS["r1-n8-k4-v32000-f32"].scaled(R=2, V=1000, ld=1008)
    g = synth.make_gumbel(w, 4)
    assert g.shape == (2, 8, 1008) and torch.all(g[..., 1000:] == 8192.0)
    assert abs(float(g[..., :1000].mean()) - 0.5772) < 0.02    # the Gumbel mean
    assert torch.equal(g, synth.make_gumbel(w, 4))
