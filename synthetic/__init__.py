"""Seeded synthetic decode workloads.

This module only draws inputs: queries, paged K/V caches, block tables, sequence
lengths and the projection basis P.  It holds none of the method's arithmetic,
so both the HIP path and the CPU oracle can be fed from it.

The shapes and value distributions stand in for the long-context decode
workloads the pages evaluate on (Llama-3.1-8B-class GQA models on RULER,
LongBench, Loogle and AIME2024 generations of up to 32K tokens; edgentiq blog
post "vAttention: a new approach to sparse attention with guaranteed accuracy",
section "Performance and Efficiency").  None of those models or datasets is
used: every tensor is drawn from a seeded torch generator.

Layouts (all contiguous, host tensors):
  q            [B, Hq, d]                    float32
  k_cache      [num_blocks, Hkv, 16, d]      bfloat16 or float32
  v_cache      [num_blocks, Hkv, 16, d]      same dtype as k_cache
  block_table  [B, max_blocks]               int32 (page ids, -1 unused)
  seq_lens     [B]                           int32
  proj         [d, r] or [Hkv, d, r]         float32, orthonormal columns (one basis, or one per KV head)
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

PAGE = 16


@dataclass
class Workload:
    name: str
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_table: torch.Tensor
    seq_lens: torch.Tensor
    proj: torch.Tensor | None
    cfg: dict
    max_seq_len: int
    meta: dict = field(default_factory=dict)

    @property
    def B(self):
        return self.q.shape[0]

    @property
    def Hq(self):
        return self.q.shape[1]

    @property
    def d(self):
        return self.q.shape[2]

    @property
    def Hkv(self):
        return self.k_cache.shape[1]

    def heads_tokens(self) -> int:
        """Logical context coverage of one decode step: sum_b Hq * L_b."""
        return int(self.Hq * int(self.seq_lens.sum()))

    def oracle_arrays(self):
        """numpy views for the oracle: bf16 caches as uint16 bit patterns."""
        def kv(t):
            if t.dtype == torch.bfloat16:
                return t.view(torch.int16).numpy().view("uint16")
            return t.numpy()
        return dict(q=self.q.numpy(), k_cache=kv(self.k_cache), v_cache=kv(self.v_cache),
                    block_table=self.block_table.numpy(), seq_lens=self.seq_lens.numpy(),
                    proj=None if self.proj is None else self.proj.numpy(),
                    max_seq_len=self.max_seq_len)


def orthonormal(rows: int, cols: int, gen: torch.Generator) -> torch.Tensor:
    """Q factor of a seeded Gaussian matrix (columns orthonormal)."""
    a = torch.randn(rows, cols, generator=gen, dtype=torch.float64)
    qm, rm = torch.linalg.qr(a)
    qm = qm * torch.sign(torch.diagonal(rm)).unsqueeze(0)
    return qm.to(torch.float32).contiguous()


def _block_table(seq_lens, max_seq_len, shuffle, gen):
    B = len(seq_lens)
    max_blocks = max(1, -(-max_seq_len // PAGE))
    need = [-(-L // PAGE) for L in seq_lens]
    total = sum(need)
    ids = torch.arange(total, dtype=torch.int64)
    if shuffle:
        ids = ids[torch.randperm(total, generator=gen)]
    bt = torch.full((B, max_blocks), -1, dtype=torch.int32)
    off = 0
    for b in range(B):
        bt[b, :need[b]] = ids[off:off + need[b]].to(torch.int32)
        off += need[b]
    return bt, max(total, 1)


def _to_paged(rows, bt, seq_lens, num_blocks, dtype):
    """rows: list over b of [Hkv, L_b, d] float32 -> [num_blocks, Hkv, 16, d]."""
    Hkv, d = rows[0].shape[0], rows[0].shape[2]
    cache = torch.zeros(num_blocks, Hkv, PAGE, d, dtype=torch.float32)
    for b, L in enumerate(seq_lens):
        nb = -(-L // PAGE)
        if nb == 0:
            continue
        x = torch.zeros(Hkv, nb * PAGE, d)
        x[:, :L] = rows[b]
        x = x.view(Hkv, nb, PAGE, d).permute(1, 0, 2, 3)
        cache[bt[b, :nb].long()] = x
    return cache.to(dtype).contiguous()


def make(*, name="custom", B=1, Hq=4, Hkv=4, d=64, seq_lens=(1024,), kv_dtype="f32",
         recipe="normal", rank=32, predictor=1, sinks=4, window=32, topk_abs=-1,
         topk_ppm=25000, base_ppm=50000, force_budget=-1, eps=0.05, delta=0.05, seed=0,
         data_seed=1000, shuffle=False, q_std=1.0, k_std=1.0, planted=8, plant_scale=4.0,
         outlier_channels=4, outlier_scale=8.0, lowrank_dim=24, lowrank_noise=0.1,
         peaked_frac=0.5, hidden_logit=40.0, max_seq_len=None, proj_per_head=False, v_mean=0.0,
         guarantee=0) -> Workload:
    """Draw one workload.

    recipe:
      normal    q, K, V ~ N(0, 1) (scaled by q_std / k_std)
      planted   as normal, plus `planted` heavy-hitter keys per query head:
                K = plant_scale * q_hat + N(0, I) at distinct uniform positions
      outlier   K ~ N(0,1) with `outlier_channels` channels per KV head scaled
                by `outlier_scale`
      flat      q, K ~ N(0, q_std^2), N(0, k_std^2) (use 0.3 for near-uniform softmax)
      lowrank   K = Z U^T + N(0, lowrank_noise^2), U a d x lowrank_dim orthonormal
                basis per KV head, Z ~ N(0, I)
      mixed     per (b, KV head) a seeded coin: `planted` or `flat` (k_std=q_std=0.3)

    v_mean: values V = v_mean * mu_g + N(0, I), with mu_g ~ N(0, I) drawn once
    per KV head (a shared direction, as values of real heads have; 0 gives
    zero-mean values whose attention output nearly cancels).
    guarantee: 0 the denominator only, 1 the denominator and the numerator.
      hidden    as normal, plus keys the low-rank predictor cannot see: for every
                query head h one key c * u / |u| with u = q_h - P P^T q_h (the
                part of q_h outside the predictor's span), so its predicted score
                is ~0 while its scaled score q_h . K / sqrt(d) is `hidden_logit`;
                and, when G >= 2, one key that adds to head 0's hidden direction
                a component along P P^T q_1, which puts it among head 1's
                predicted top scores (a base-pass member of the group) while it
                stays outside head 0's fixed set.  Positions are uniform in the
                middle half of each sequence.  LOWRANK predictor only.
    """
    gen = torch.Generator().manual_seed(int(data_seed))
    seq_lens = [int(x) for x in seq_lens]
    assert len(seq_lens) == B and Hq % Hkv == 0
    G = Hq // Hkv
    msl = max(seq_lens) if max_seq_len is None else int(max_seq_len)
    bt, num_blocks = _block_table(seq_lens, msl, shuffle, gen)

    q = torch.randn(B, Hq, d, generator=gen) * q_std
    rows_k, rows_v = [], []
    kinds = []
    plants = []
    outlier_idx = None
    if recipe == "outlier":
        outlier_idx = torch.stack([torch.randperm(d, generator=gen)[:outlier_channels]
                                   for _ in range(Hkv)])
    assert predictor != 2 or rank == 32, "signatures have 32 bits"
    hidden_proj = None
    if recipe == "hidden":
        assert predictor == 1
        hidden_proj = orthonormal(d, rank, gen)
    U = None
    if recipe == "lowrank":
        U = torch.stack([orthonormal(d, lowrank_dim, gen) for _ in range(Hkv)])
    # the value means come from a generator of their own, so every other
    # tensor of the workload is the same for any v_mean
    v_mu = (torch.randn(Hkv, 1, d, generator=torch.Generator().manual_seed(int(data_seed) + 7919)) * v_mean
            if v_mean else None)
    for b, L in enumerate(seq_lens):
        v = torch.randn(Hkv, L, d, generator=gen)
        if v_mu is not None:
            v = v + v_mu
        if recipe in ("normal", "planted", "hidden"):
            k = torch.randn(Hkv, L, d, generator=gen) * k_std
        elif recipe == "flat":
            k = torch.randn(Hkv, L, d, generator=gen) * k_std
        elif recipe == "outlier":
            k = torch.randn(Hkv, L, d, generator=gen)
            for g in range(Hkv):
                k[g][:, outlier_idx[g]] *= outlier_scale
        elif recipe == "lowrank":
            z = torch.randn(Hkv, L, lowrank_dim, generator=gen)
            k = torch.einsum("glr,gdr->gld", z, U) + \
                torch.randn(Hkv, L, d, generator=gen) * lowrank_noise
        elif recipe == "mixed":
            k = torch.empty(Hkv, L, d)
            coins = torch.rand(Hkv, generator=gen) < peaked_frac
            for g in range(Hkv):
                if coins[g]:
                    k[g] = torch.randn(L, d, generator=gen)
                    kinds.append((b, g, "peaked"))
                else:
                    k[g] = torch.randn(L, d, generator=gen) * 0.3
                    q[b, g * G:(g + 1) * G] = torch.randn(G, d, generator=gen) * 0.3
                    kinds.append((b, g, "flat"))
        else:
            raise ValueError(recipe)
        plant_groups = []
        if recipe == "planted":
            plant_groups = list(range(Hkv))
        elif recipe == "mixed":
            plant_groups = [g for (bb, g, kind) in kinds if bb == b and kind == "peaked"]
        for g in (plant_groups if planted > 0 else []):
            n_pl = min(planted * G, L)
            pos = torch.randperm(L, generator=gen)[:n_pl]
            for j in range(n_pl):
                h = g * G + (j // planted) % G
                qh = q[b, h] / q[b, h].norm()
                k[g, pos[j]] = plant_scale * qh + torch.randn(d, generator=gen)
                plants.append((b, h, int(pos[j])))
        if recipe == "hidden" and L >= 8:
            Pm = hidden_proj.double()
            for g in range(Hkv):
                pos = (L // 4 + torch.randperm(max(L // 2, 1), generator=gen)[:G + 1]).tolist()
                for hh in range(G):
                    qh = q[b, g * G + hh].double()
                    u = qh - Pm @ (Pm.T @ qh)
                    c = hidden_logit * math.sqrt(d) / float(u.norm())
                    k[g, pos[hh]] = (c * u / u.norm()).float()
                    plants.append((b, g * G + hh, int(pos[hh])))
                if G >= 2:
                    q0, q1 = q[b, g * G].double(), q[b, g * G + 1].double()
                    u = q0 - Pm @ (Pm.T @ q0)
                    w = Pm @ (Pm.T @ q1)
                    kk = hidden_logit * math.sqrt(d) / float(u.norm()) * u / u.norm() + 40.0 * w / w.norm()
                    k[g, pos[G]] = kk.float()
                    plants.append((b, g * G, int(pos[G])))
        rows_k.append(k)
        rows_v.append(v)

    dt = torch.bfloat16 if kv_dtype == "bf16" else torch.float32
    k_cache = _to_paged(rows_k, bt, seq_lens, num_blocks, dt)
    v_cache = _to_paged(rows_v, bt, seq_lens, num_blocks, dt)
    if hidden_proj is not None:
        proj = hidden_proj
    elif predictor in (1, 2) and proj_per_head:  # a seeded orthonormal basis for every KV head
        proj = torch.stack([orthonormal(d, rank, gen) for _ in range(Hkv)])
    else:
        # predictor 2: the 32 hyperplanes of the signatures (random directions,
        # taken orthonormal like the low-rank basis)
        proj = orthonormal(d, rank, gen) if predictor in (1, 2) else None
    cfg = dict(sinks=sinks, window=window, topk_abs=topk_abs, topk_ppm=topk_ppm,
               base_ppm=base_ppm, force_budget=force_budget, predictor=predictor,
               rank=rank if predictor in (1, 2) else 0, eps=eps, delta=delta, seed=seed, guarantee=guarantee)
    return Workload(name=name, q=q.contiguous(), k_cache=k_cache, v_cache=v_cache,
                    block_table=bt, seq_lens=torch.tensor(seq_lens, dtype=torch.int32),
                    proj=proj, cfg=cfg, max_seq_len=msl, meta=dict(kinds=kinds, recipe=recipe, plants=plants))


# ---------------------------------------------------------------------------
# The five named workloads (the full-size shapes), with optional shrinking for
# parity tests: `scale_len` divides the context lengths, `batch` overrides B.
# ---------------------------------------------------------------------------

def tiny(seed=0, **kw):
    """B1, 4 q / 4 KV heads, d64, L1024, fp32 KV, 8 planted heavy hitters per
    head, exact-score (oracle) top-k 32, sinks 4, window 32, eps=delta=0.05."""
    args = dict(name="tiny_1k", B=1, Hq=4, Hkv=4, d=64, seq_lens=(1024,), kv_dtype="f32",
                recipe="planted", predictor=0, sinks=4, window=32, topk_abs=32, eps=0.05,
                delta=0.05, seed=seed, data_seed=1001)
    args.update(kw)
    return make(**args)


def llama8b_32k(seed=0, B=8, L=32768, shuffle=False, **kw):
    """Llama-3-8B-shaped layer: B8, 32 q / 8 KV heads, d128, L32768, bf16 KV;
    K ~ N(0,1) with 4 of 128 channels scaled x8; low-rank predictor r=32 from
    a fixed random orthonormal P; sinks 128, window 128, top-k 2.5%; base
    sample 10% of the tail (the smallest of 5, 10 and 20% at which the measured
    (eps, delta) rate of this workload stays below delta; 5% does not)."""
    args = dict(name="llama8b_32k", B=B, Hq=32, Hkv=8, d=128, seq_lens=(L,) * B,
                kv_dtype="bf16", recipe="outlier", predictor=1, rank=32, sinks=128,
                window=128, topk_ppm=25000, base_ppm=100000, eps=0.05, delta=0.05, seed=seed,
                data_seed=1002, shuffle=shuffle)
    args.update(kw)
    return make(**args)


def flat_128k(seed=0, L=131072, **kw):
    """B1, 32 q / 8 KV heads, d128, L131072, bf16; q, K ~ N(0, 0.3^2);
    sinks 128, window 128, top-k 1%, eps 0.02, delta 0.05."""
    args = dict(name="flat_128k", B=1, Hq=32, Hkv=8, d=128, seq_lens=(L,), kv_dtype="bf16",
                recipe="flat", q_std=0.3, k_std=0.3, predictor=1, rank=32, sinks=128,
                window=128, topk_ppm=10000, eps=0.02, delta=0.05, seed=seed, data_seed=1003)
    args.update(kw)
    return make(**args)


def ragged_b64(seed=0, B=64, lo=1024, hi=16384, **kw):
    """B64, L_b ~ U{1024..16384}, 32 q / 8 KV heads, d128, bf16, shuffled
    block table; per (b, KV head) planted-peaked or flat; sinks 64, window 64,
    top-k 2%, eps 0.05, delta 0.1."""
    g = torch.Generator().manual_seed(2004)
    lens = torch.randint(lo, hi + 1, (B,), generator=g).tolist()
    args = dict(name="ragged_b64", B=B, Hq=32, Hkv=8, d=128, seq_lens=lens, kv_dtype="bf16",
                recipe="mixed", predictor=1, rank=32, sinks=64, window=64, topk_ppm=20000,
                eps=0.05, delta=0.1, seed=seed, data_seed=1004, shuffle=True)
    args.update(kw)
    return make(**args)


def wide_gqa_64k(seed=0, eps=0.05, B=4, L=65536, **kw):
    """70B-shaped: B4, 64 q / 8 KV heads (8:1), d128, L65536, bf16; keys of
    effective rank 24 plus N(0, 0.1^2); r=32 predictor; sinks/window 128,
    top-k 2.5%; eps swept over {0.01, 0.02, 0.05, 0.1}, delta 0.05."""
    args = dict(name="wide_gqa_64k", B=B, Hq=64, Hkv=8, d=128, seq_lens=(L,) * B,
                kv_dtype="bf16", recipe="lowrank", predictor=1, rank=32, sinks=128,
                window=128, topk_ppm=25000, eps=eps, delta=0.05, seed=seed, data_seed=1005)
    args.update(kw)
    return make(**args)


def repaged(w: Workload, seed: int = 0) -> Workload:
    """The same workload with its cache pages moved to a seeded permutation of
    the physical page ids and the block table rewritten to match: every token's
    K and V (and so every result) are unchanged, only the physical layout of
    the cache differs."""
    import dataclasses
    gen = torch.Generator().manual_seed(seed)
    perm = torch.randperm(w.k_cache.shape[0], generator=gen)  # new id of page p
    k = torch.empty_like(w.k_cache)
    v = torch.empty_like(w.v_cache)
    k[perm] = w.k_cache
    v[perm] = w.v_cache
    bt = w.block_table.clone()
    used = bt >= 0
    bt[used] = perm[bt[used].long()].to(torch.int32)
    return dataclasses.replace(w, name=w.name + "_repaged", k_cache=k, v_cache=v, block_table=bt)


WORKLOADS = {"tiny_1k": tiny, "llama8b_32k": llama8b_32k, "flat_128k": flat_128k,
             "ragged_b64": ragged_b64, "wide_gqa_64k": wide_gqa_64k}
