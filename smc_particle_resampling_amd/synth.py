"""Seeded synthetic inputs for one SMC-SD round.

The round's inputs are the outputs of model forward passes that this library does not run:
drafted tokens, target and draft logits over the full vocabulary, plus precomputed Gumbel
noise, one uniform per request and the paged-KV page table. This module draws them from
seeded ``torch.Generator`` streams with the shapes and value distributions of the workloads
below. It holds none of the round's arithmetic; the GPU library and the CPU oracle both
consume what it produces.

Recipe (every tensor from its own stream, ``seed * 1000 + stream id``; logits drawn in fp32
and rounded to bf16 with round-to-nearest-even where the workload is bf16):
  * target rows (positions 0..K, row K is the bonus position):
      "normal": Normal(0, sigma^2), then ``n_peaks`` ids per row drawn uniformly (repeats
                collapse) are raised by ``peak_boost``;
      "zipf":   -alpha * ln(rank) + Normal(0, sigma^2), rank a seeded permutation per row.
  * draft rows (positions 0..K-1):
      "normal": target row + Normal(0, draft_sigma^2);
      "zipf":   an independent Zipf row whose ``shared_top`` best ids (in order) equal the
                target row's, the remaining ranks an independent permutation.
  * drafted token x_k: one draw from softmax(draft row k / T) (torch.multinomial).
  * bonus noise: standard Gumbel -log(-log U), U uniform clamped into (0, 1), fp32.
  * uniform: one U[0,1) per request; temperatures per workload; log-weights -log N.
  * page table [R,N,P]: the first P/2 columns are prompt pages shared by all N particles;
    each later column first copies every particle's earlier columns from an ancestor drawn
    uniformly, then gives each particle a fresh page; ids are finally mapped through a
    seeded permutation of the pool; refcount = number of table entries naming each page.
  * page pool between rounds (make_page_pool): per request a length drawn uniformly, its
    columns grown with the same genealogy, then one last uniform draw of ancestors (as a
    resampling step leaves them, duplicates sharing every page, tail included); pages the
    draws dropped keep refcount 0, ``spare`` more pages sit on the free list (refcount -1)
    in a seeded order; KV bytes uniform.
"""
from __future__ import annotations

import dataclasses
import math

import torch

STREAMS = dict(target=1, peaks=2, draft=3, tokens=4, gumbel=5, uniform=6, temp=7, pages=8,
               ragged=9, zipf_q=10, potential=11, accept=12, residual=13, pool=14, kv=15,
               ancestors=16, noise=17)


@dataclasses.dataclass(frozen=True)
class Workload:
    """Sizes and value distributions of one synthetic round."""
    name: str
    R: int
    N: int
    K: int
    V: int
    dtype: str = "bf16"            # "bf16" or "f32"
    target: str = "normal"         # "normal" or "zipf"
    sigma: float = 3.0             # target noise std
    n_peaks: int = 0               # normal: peak ids per row
    peak_boost: float = 8.0
    zipf_alpha: float = 1.1
    shared_top: int = 20           # zipf: top ids shared by draft and target
    draft_sigma: float = 1.0       # normal: draft = target + Normal(0, draft_sigma^2)
    temps: tuple = (1.0,)          # one value, or a set drawn uniformly per request
    ctx: int = 512                 # context tokens per particle
    page_size: int = 16
    mode: str = "always"           # resample "always" | "ess" | "never"
    ess_frac: float = 0.5
    tv: bool = False
    ld: int | None = None          # row stride in elements (default: V rounded up to 16 B)

    @property
    def P(self) -> int:
        return max(1, self.ctx // self.page_size)

    @property
    def row_stride(self) -> int:
        if self.ld is not None:
            return self.ld
        per16 = 4 if self.dtype == "f32" else 8
        return -(-self.V // per16) * per16

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def algorithmic_bytes(self) -> dict:
        """Bytes a round must move at least once: every logit read once, the bonus noise,
        page-table rows in and out."""
        R, N, K, V = self.R, self.N, self.K, self.V
        e = self.elem_bytes
        return dict(target=R * N * (K + 1) * V * e, draft=R * N * K * V * e,
                    noise=R * N * V * 4, table=2 * R * N * self.P * 4)

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads the round is measured and checked on; named by what they are.
WORKLOADS = {
    "r1-n8-k4-v32000-f32": Workload(
        "r1-n8-k4-v32000-f32", R=1, N=8, K=4, V=32000, dtype="f32", sigma=2.0, n_peaks=0,
        draft_sigma=0.5, temps=(1.0,), ctx=512, mode="always"),
    "r16-n16-k4-v128256-bf16": Workload(
        "r16-n16-k4-v128256-bf16", R=16, N=16, K=4, V=128256, sigma=3.0, n_peaks=50,
        draft_sigma=0.7, temps=(0.7,), ctx=2048, mode="always"),
    "r64-n32-k8-v128256-bf16-tv": Workload(
        "r64-n32-k8-v128256-bf16-tv", R=64, N=32, K=8, V=128256, sigma=3.0, n_peaks=50,
        draft_sigma=1.5, temps=(1.0,), ctx=4096, mode="always", tv=True),
    "r8-n16-k4-v152064-bf16-zipf-ess": Workload(
        "r8-n16-k4-v152064-bf16-zipf-ess", R=8, N=16, K=4, V=152064, target="zipf",
        sigma=0.3, zipf_alpha=1.1, shared_top=20, temps=(1.0,), ctx=32768, mode="ess",
        ess_frac=0.5),
    "r32-n32-k8-v256000-bf16-tv-mixT": Workload(
        "r32-n32-k8-v256000-bf16-tv-mixT", R=32, N=32, K=8, V=256000, sigma=3.0, n_peaks=100,
        draft_sigma=1.0, temps=(0.6, 0.8, 1.0, 1.2), ctx=8192, mode="always", tv=True),
}
HEADLINE = "r64-n32-k8-v128256-bf16-tv"


def _gen(seed: int, stream: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000 + STREAMS[stream])
    return g


def _store(x: torch.Tensor, w: Workload) -> torch.Tensor:
    return x.to(torch.bfloat16) if w.dtype == "bf16" else x.to(torch.float32)


def _zipf_rows(n_rows: int, w: Workload, g: torch.Generator, device, rank_ids=None):
    """Rows of -alpha*ln(rank) + noise. Returns (logits fp32 [n_rows, V], ids by rank)."""
    V = w.V
    if rank_ids is None:
        rank_ids = torch.argsort(torch.rand(n_rows, V, generator=g, device=device), dim=1)
    ranks = torch.empty_like(rank_ids)
    ar = torch.arange(1, V + 1, device=device).expand(n_rows, V)
    ranks.scatter_(1, rank_ids, ar)
    z = -w.zipf_alpha * torch.log(ranks.to(torch.float32))
    z = z + w.sigma * torch.randn(n_rows, V, generator=g, device=device)
    return z, rank_ids


def _rows_normal(n_rows, w, g_main, g_peaks, device):
    z = w.sigma * torch.randn(n_rows, w.V, generator=g_main, device=device)
    if w.n_peaks > 0:
        idx = torch.randint(0, w.V, (n_rows, w.n_peaks), generator=g_peaks, device=device)
        boost = torch.zeros_like(z)
        boost.scatter_(1, idx, w.peak_boost)
        z = z + boost
    return z


def make_log_potential(R: int, N: int, seed: int, device="cpu", p_removed: float = 0.1):
    """Per-particle log potentials [R, N] float32: N(0, 1), with a fraction of particles
    removed (-inf), always keeping at least one finite particle per request."""
    g = _gen(seed, "potential", device)
    lp = torch.randn((R, N), generator=g, device=device, dtype=torch.float32)
    removed = torch.rand((R, N), generator=g, device=device) < p_removed
    removed[:, 0] = False
    return lp.masked_fill(removed, float("-inf"))


def make_verify_uniforms(R: int, N: int, K: int, seed: int, device="cpu") -> dict:
    """Uniforms of speculative-decoding verification: accept_uniform [R, N, K] and
    residual_uniform [R, N], float32 in [0, 1)."""
    return dict(
        accept_uniform=torch.rand((R, N, K), generator=_gen(seed, "accept", device),
                                  device=device, dtype=torch.float32),
        residual_uniform=torch.rand((R, N), generator=_gen(seed, "residual", device),
                                    device=device, dtype=torch.float32))


def topk_rows(inputs: dict):
    """Gumbel-Top-K drafting inputs from a round's inputs: every particle's first target row
    as a [R*N, ld] logits matrix, its noise row, and the request temperature per row."""
    R, N, _, ld = inputs["target"].shape
    return (inputs["target"][:, :, 0].contiguous().view(R * N, ld),
            inputs["temperature"].repeat_interleave(N).contiguous(),
            inputs["gumbel"].view(R * N, ld))


def make_page_table(R: int, N: int, P: int, seed: int, ragged: bool = False):
    """Page table [R,N,P] int32 (negative = unused), refcount, num_pages (CPU tensors)."""
    g = _gen(seed, "pages", "cpu")
    half = P // 2
    table = torch.full((R, N, P), -1, dtype=torch.int64)
    nxt = 0
    prompt = torch.arange(R * half, dtype=torch.int64).view(R, 1, half)
    table[:, :, :half] = prompt
    nxt = R * half
    for c in range(half, P):
        if c > half:
            a = torch.randint(0, N, (R, N), generator=g)
            table[:, :, :c] = torch.gather(table[:, :, :c], 1, a[:, :, None].expand(R, N, c))
        table[:, :, c] = torch.arange(nxt, nxt + R * N, dtype=torch.int64).view(R, N)
        nxt += R * N
    num_pages = nxt + max(16, nxt // 16)      # pool with some never-used pages
    perm = torch.randperm(num_pages, generator=g)
    table = perm[table]
    if ragged:
        gr = _gen(seed, "ragged", "cpu")
        lengths = torch.randint(half, P + 1, (R, N), generator=gr)
        col = torch.arange(P).view(1, 1, P)
        table = torch.where(col < lengths[:, :, None], table, torch.full_like(table, -1))
    table = table.to(torch.int32)
    valid = table[table >= 0].to(torch.int64)
    refcount = torch.bincount(valid, minlength=num_pages).to(torch.int32)
    return table.contiguous(), refcount.contiguous(), int(num_pages)


def make_gumbel(w: Workload, seed: int, device="cpu", pad_value: float = 8192.0) -> torch.Tensor:
    """[R,N,ld] float32 standard Gumbel noise alone (say, the fresh noise of a bonus drawn
    after resampling), drawn as the round's noise from its own stream; padding pad_value."""
    R, N, V, ld = w.R, w.N, w.V, w.row_stride
    dev = torch.device(device)
    out = torch.full((R, N, ld), pad_value, dtype=torch.float32, device=dev)
    g = _gen(seed, "noise", dev)
    tiny = torch.finfo(torch.float32).tiny
    for r in range(R):
        u = torch.rand(N, V, generator=g, device=dev).clamp_(tiny, 1.0 - 2.0 ** -24)
        out[r, :, :V] = -torch.log(-torch.log(u))
    return out


def make_ancestors(R: int, N: int, seed: int, device="cpu") -> torch.Tensor:
    """[R,N] int32 ancestor indices as a resampling step leaves them: N uniform draws from
    [0, N) per request, sorted."""
    g = _gen(seed, "ancestors", "cpu")
    a = torch.sort(torch.randint(0, N, (R, N), generator=g), dim=1).values
    return a.to(torch.int32).to(device)


def make_page_pool(R: int, N: int, P: int, page_size: int, seed: int, steps=None,
                   spare: int = 64, kv_count: int = 0, page_bytes: int = 0,
                   min_len: int = 1) -> dict:
    """A consistent paged-KV pool between two rounds, as CPU tensors: page_table [R,N,P]
    int32 (-1 past each request's length), refcount [num_pages] (-1 = free, else the
    entries naming the page; pages dropped by the genealogy hold 0), free_ids [num_pages]
    (the free pages at [0, n_free), the rest -7), n_free, len_before and len_after [R]
    (len_after = len_before + steps[r]; steps default: uniform in [0, 2 * page_size]), kv
    [kv_count, num_pages, page_bytes] uint8 or None."""
    g = _gen(seed, "pool", "cpu")
    if steps is None:
        steps = torch.randint(0, 2 * page_size + 1, (R,), generator=g)
    steps = torch.as_tensor(steps, dtype=torch.int64).expand(R).clone()
    cap = P * page_size
    if int(steps.max()) + min_len > cap:
        raise ValueError("steps do not fit P * page_size")
    hi = cap - steps
    len_before = torch.stack([torch.randint(min_len, int(h) + 1, (1,), generator=g)[0]
                              for h in hi])
    tables = []
    nxt = 0
    for r in range(R):
        nc = -(-int(len_before[r]) // page_size)
        t = torch.full((N, P), -1, dtype=torch.int64)
        for c in range(nc):
            if c == 0:
                t[:, 0] = nxt                         # prompt page shared by every particle
                nxt += 1
                continue
            a = torch.randint(0, N, (N,), generator=g)
            t[:, :c] = t[a, :c]
            t[:, c] = torch.arange(nxt, nxt + N)
            nxt += N
        a = torch.randint(0, N, (N,), generator=g)
        tables.append(t[a])
    table = torch.stack(tables) if R else torch.full((0, N, P), -1, dtype=torch.int64)
    num_pages = nxt + spare
    perm = torch.randperm(num_pages, generator=g)
    table = torch.where(table >= 0, perm[table.clamp(min=0)], table).to(torch.int32)
    valid = table[table >= 0].to(torch.int64)
    refcount = torch.bincount(valid, minlength=num_pages).to(torch.int32)
    free = perm[nxt:].to(torch.int32)                 # never referenced: on the free list
    refcount[free.long()] = -1
    free_ids = torch.full((num_pages,), -7, dtype=torch.int32)
    free_ids[:spare] = free
    kv = None
    if kv_count:
        gk = _gen(seed, "kv", "cpu")
        kv = torch.randint(0, 256, (kv_count, num_pages, page_bytes), generator=gk,
                           dtype=torch.int32).to(torch.uint8)
    return dict(page_table=table.contiguous(), refcount=refcount, free_ids=free_ids,
                n_free=spare, len_before=len_before.to(torch.int32),
                len_after=(len_before + steps).to(torch.int32), kv=kv, page_size=page_size)


@torch.no_grad()
def make_inputs(w: Workload, seed: int = 0, device="cpu", pages: bool = True,
                ragged_pages: bool = False, pad_value: float = 8192.0) -> dict:
    """All inputs of one round as torch tensors on ``device``.

    Rows are padded to ``w.row_stride`` elements; padding columns hold ``pad_value`` (large,
    so a kernel that read past V would be caught by the parity tests)."""
    R, N, K, V = w.R, w.N, w.K, w.V
    ld = w.row_stride
    dev = torch.device(device)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    target = torch.full((R, N, K + 1, ld), pad_value, dtype=tdt, device=dev)
    draft = torch.full((R, N, K, ld), pad_value, dtype=tdt, device=dev)
    gumbel = torch.full((R, N, ld), pad_value, dtype=torch.float32, device=dev)
    tokens = torch.empty((R, N, K), dtype=torch.int32, device=dev)

    gt = _gen(seed, "target", dev)
    gp = _gen(seed, "peaks", dev)
    gd = _gen(seed, "draft", dev)
    gk = _gen(seed, "tokens", dev)
    gg = _gen(seed, "gumbel", dev)
    gz = _gen(seed, "zipf_q", dev)

    if len(w.temps) == 1:
        temperature = torch.full((R,), float(w.temps[0]), dtype=torch.float32, device=dev)
    else:
        choice = torch.randint(0, len(w.temps), (R,), generator=_gen(seed, "temp", dev),
                               device=dev)
        temperature = torch.tensor(w.temps, dtype=torch.float32, device=dev)[choice]

    tiny = torch.finfo(torch.float32).tiny
    for r in range(R):            # one request at a time keeps temporaries small
        n_rows_t = N * (K + 1)
        if w.target == "zipf":
            zt, ids = _zipf_rows(n_rows_t, w, gt, dev)
            ids = ids.view(N, K + 1, V)[:, :K].reshape(N * K, V)
            # draft: same top ids in the same order, the rest independently permuted
            rest = ids[:, w.shared_top:]
            shuffle = torch.argsort(torch.rand(rest.shape, generator=gz, device=dev), dim=1)
            q_ids = torch.cat([ids[:, :w.shared_top], torch.gather(rest, 1, shuffle)], dim=1)
            zq, _ = _zipf_rows(N * K, w, gd, dev, rank_ids=q_ids)
        else:
            zt = _rows_normal(n_rows_t, w, gt, gp, dev)
            zq = zt.view(N, K + 1, V)[:, :K].reshape(N * K, V)
            zq = zq + w.draft_sigma * torch.randn(N * K, V, generator=gd, device=dev)
        zt_s = _store(zt, w)
        zq_s = _store(zq, w)
        target[r, :, :, :V] = zt_s.view(N, K + 1, V)
        draft[r, :, :, :V] = zq_s.view(N, K, V)
        # drafted tokens: one draw per row from the draft's tempered softmax
        probs = torch.softmax(zq_s.to(torch.float32) / temperature[r], dim=1)
        tokens[r] = torch.multinomial(probs, 1, generator=gk).view(N, K).to(torch.int32)
        u = torch.rand(N, V, generator=gg, device=dev).clamp_(tiny, 1.0 - 2.0 ** -24)
        gumbel[r, :, :V] = -torch.log(-torch.log(u))

    uniform = torch.rand(R, generator=_gen(seed, "uniform", dev), device=dev).to(torch.float32)
    log_weights = torch.full((R, N), -math.log(N), dtype=torch.float32, device=dev)
    out = dict(target=target, draft=draft, tokens=tokens, temperature=temperature,
               gumbel=gumbel, uniform=uniform, log_weights=log_weights, V=V, ld=ld)
    if pages:
        pt, rc, npg = make_page_table(R, N, w.P, seed, ragged=ragged_pages)
        out.update(page_table=pt.to(dev), refcount=rc.to(dev), num_pages=npg)
    return out


def to_host(inputs: dict, requests=None) -> dict:
    """numpy views for the oracle: bf16 as raw uint16 bits; optionally a subset of requests
    (page tables and refcounts are per-request independent only if page ids are disjoint,
    which holds for make_page_table)."""
    import numpy as np
    sel = slice(None) if requests is None else torch.as_tensor(requests, dtype=torch.long)

    def host(t, per_request=True):
        t = t[sel.to(t.device)] if (per_request and not isinstance(sel, slice)) else t
        t = t.detach().cpu().contiguous()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.numpy()

    out = {k: host(inputs[k]) for k in ("target", "draft", "tokens", "temperature", "gumbel",
                                         "uniform", "log_weights")}
    for k in ("log_potential", "accept_uniform", "residual_uniform"):
        if inputs.get(k) is not None:
            out[k] = host(inputs[k])
    if "page_table" in inputs:
        out["page_table"] = host(inputs["page_table"])
        out["refcount"] = host(inputs["refcount"], per_request=False)
    out["V"] = inputs["V"]
    return out
