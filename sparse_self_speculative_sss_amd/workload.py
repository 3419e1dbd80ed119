"""Seeded synthetic inputs shaped like the pages' decode workloads.

This module draws random numbers and lays them out as a paged KV cache; it
contains none of the attention arithmetic.  Both the HIP path and the CPU
oracle consume what it produces.

Shapes follow the pages' workloads: Qwen3-8B has 32 query heads, 8 KV heads
and head dimension 128 (SparseSpec §5.1); batch 128 with 8K-token outputs is
the KV-loading example of SparseSpec's introduction; the draft budget of 5%
of the KV and draft length k come from SparseSpec §5.4.  No dataset item is
used: every value is drawn from a seeded generator.

Recipe (per workload, one ``torch.Generator`` seeded with ``seed``; the draw
order below is fixed):

1. sequence lengths (fixed, or uniform integers in [lo, hi]); for the mixed
   batch also the per-request verify flag (verify with probability p);
2. page table: the pool of sum_b ceil(L_b / P) pages is randomly permuted and
   handed out request by request (identity for the contiguous case);
3. queries, then K, then V, iid N(0, sigma^2) in fp32, rounded once to the
   cache dtype (bf16 round-to-nearest-even);
4. planted heavy hitters per (request, KV head): u = mean of the group's
   query rows normalised, lambda = 4 sqrt(d) / |mean|, so that the mean query
   gains +4 nats of logit on each planted key (k <- k + lambda u, rounded
   again); positions are distinct draws below the window start, or whole
   blocks in contiguous clusters;
5. for mixed-batch draft requests, a random sorted set of distinct candidate
   blocks of the requested budget;
6. for sparse verification (``layout_shared`` set), a layout per (verify
   request, KV head, query position): N = the block budget, of which
   round(layout_shared * N) blocks are common to every position of the unit
   (blocks holding planted keys first, in random order, then other random
   candidates) and the rest are drawn per position; entries shuffled, -1
   padded.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import torch


@dataclass(frozen=True)
class Shape:
    name: str
    B: int
    L: object                    # int, or (lo, hi) inclusive uniform
    Hq: int
    Hkv: int
    d: int
    dtype: str                   # "f32" or "bf16"
    n_q: int                     # k + 1 verify queries
    block_size: int
    page_size: int
    window: int
    budget: Optional[int] = None          # fixed N blocks
    budget_frac: Optional[float] = None   # N = ceil(frac * nblk)
    sigma: str = "inv_sqrt_d"             # "one" or "inv_sqrt_d"
    planted: tuple = ("token_frac", 0.01)
    table: str = "permuted"               # "identity" or "permuted"
    num_splits: int = 0                   # 0 = library heuristic
    p_verify: Optional[float] = None      # mixed batch: P(request verifies)
    layout_shared: Optional[float] = None  # sparse verify: shared part of the layouts


SHAPES = {
    s.name: s
    for s in [
        Shape("tiny_fp32_b1_l512", B=1, L=512, Hq=4, Hkv=1, d=64, dtype="f32", n_q=4,
              block_size=16, page_size=16, window=16, budget=8, sigma="one",
              planted=("positions", 5), table="identity"),
        Shape("qwen3_8b_layer_b16_l4096", B=16, L=4096, Hq=32, Hkv=8, d=128, dtype="bf16",
              n_q=5, block_size=16, page_size=16, window=64, budget_frac=0.05),
        Shape("decode_b128_l8192", B=128, L=8192, Hq=32, Hkv=8, d=128, dtype="bf16", n_q=5,
              block_size=16, page_size=16, window=64, budget_frac=0.05),
        Shape("mixed_b96_l1k_32k", B=96, L=(1024, 32768), Hq=32, Hkv=8, d=128, dtype="bf16",
              n_q=5, block_size=16, page_size=16, window=64, budget_frac=0.05,
              p_verify=0.2),
        Shape("longctx_b4_l128k", B=4, L=131072, Hq=32, Hkv=2, d=128, dtype="bf16", n_q=5,
              block_size=64, page_size=64, window=128, budget=16,
              planted=("block_clusters", 0.005, 2), num_splits=64),
        # single-token selection (PillarAttn's own granularity): the decode
        # shape with blocks of one token, 5% of the tokens selected
        Shape("tokensel_b128_l8192", B=128, L=8192, Hq=32, Hkv=8, d=128, dtype="bf16", n_q=5,
              block_size=1, page_size=16, window=64, budget_frac=0.05),
        # sparse verification: each of the k+1 verify positions attends to its
        # own 5% of the blocks (70% of them shared by the unit's positions)
        # plus the window
        Shape("sparsever_b128_l8192", B=128, L=8192, Hq=32, Hkv=8, d=128, dtype="bf16",
              n_q=5, block_size=16, page_size=16, window=64, budget_frac=0.05,
              layout_shared=0.7),
    ]
}
SHAPE_ORDER = list(SHAPES)


@dataclass
class Batch:
    """One sub-batch of requests that read a shared paged cache."""
    q: torch.Tensor              # [B][n][Hq][d]
    page_table: torch.Tensor     # [B][max_pages] int32
    seq_lens: torch.Tensor       # [B] int32
    budget: torch.Tensor         # [B] int32
    req_ids: list                # indices into the full batch
    sel: Optional[torch.Tensor] = None        # [B][Hkv][max_sel] int32 (given lists)
    sel_count: Optional[torch.Tensor] = None  # [B][Hkv] int32
    row_sel: Optional[torch.Tensor] = None    # [B][Hkv][n][max_sel] int32 (sparse verify)
    row_sel_count: Optional[torch.Tensor] = None  # [B][Hkv][n] int32

    @property
    def B(self) -> int:
        return int(self.q.shape[0])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max().item()) if self.B else 0


@dataclass
class Workload:
    shape: Shape
    seed: int
    k_cache: torch.Tensor        # [num_pages][Hkv][P][d]
    v_cache: torch.Tensor
    seq_lens_all: list
    verify: Optional[Batch]
    draft: Optional[Batch]
    sm_scale: float
    max_blocks: int
    max_sel: int
    extras: dict = field(default_factory=dict)


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def budget_for(shape: Shape, L: int) -> int:
    if shape.budget is not None:
        return shape.budget
    return math.ceil(shape.budget_frac * _ceil_div(L, shape.block_size))


def make(shape, seed: int = 0, device="cpu", sigma: Optional[str] = None,
         B: Optional[int] = None, L=None, window: Optional[int] = None,
         budget: Optional[int] = None, n_q: Optional[int] = None,
         Hq: Optional[int] = None, Hkv: Optional[int] = None, d: Optional[int] = None,
         dtype: Optional[str] = None, block_size: Optional[int] = None,
         page_size: Optional[int] = None, planted=None, table: Optional[str] = None,
         p_verify="keep", layout_shared="keep") -> Workload:
    """Build a workload.  ``shape`` is a Shape or a name in SHAPES; keyword
    arguments override single fields (used for reduced-size and edge cases)."""
    if isinstance(shape, str):
        shape = SHAPES[shape]
    over = {k: v for k, v in dict(sigma=sigma, B=B, L=L, window=window, n_q=n_q, Hq=Hq,
                                   Hkv=Hkv, d=d, dtype=dtype, block_size=block_size,
                                   page_size=page_size, planted=planted,
                                   table=table).items() if v is not None}
    if budget is not None:
        over["budget"] = budget
        over["budget_frac"] = None
    if p_verify != "keep":
        over["p_verify"] = p_verify
    if layout_shared != "keep":
        over["layout_shared"] = layout_shared
    shape = replace(shape, **over)
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    cpu_gen = torch.Generator()
    cpu_gen.manual_seed(seed + 7919)

    Bn, Hq_, Hkv_, d_, P = shape.B, shape.Hq, shape.Hkv, shape.d, shape.page_size
    G = Hq_ // Hkv_
    cache_dtype = torch.float32 if shape.dtype == "f32" else torch.bfloat16
    sig = 1.0 if shape.sigma == "one" else 1.0 / math.sqrt(d_)

    # 1. lengths and verify flags
    if isinstance(shape.L, tuple):
        lo, hi = shape.L
        lens = torch.randint(lo, hi + 1, (Bn,), generator=cpu_gen).tolist()
    else:
        lens = [int(shape.L)] * Bn
    if shape.p_verify is not None:
        is_verify = (torch.rand(Bn, generator=cpu_gen) < shape.p_verify).tolist()
    else:
        is_verify = [True] * Bn

    # 2. page table
    n_pages = [_ceil_div(x, P) for x in lens]
    pool = sum(n_pages)
    max_pages = max(n_pages)
    if shape.table == "identity":
        perm = torch.arange(pool, dtype=torch.int32)
    else:
        perm = torch.randperm(pool, generator=cpu_gen).to(torch.int32)
    table = torch.zeros((Bn, max_pages), dtype=torch.int32)
    off = 0
    for b, n in enumerate(n_pages):
        table[b, :n] = perm[off:off + n]
        off += n

    # 3. queries and caches
    def normal(shape_, chunk_dim0=None):
        return torch.randn(shape_, generator=gen, device=device, dtype=torch.float32) * sig

    q_full = normal((Bn, shape.n_q, Hq_, d_)).to(cache_dtype)
    q_draft_own = normal((Bn, 1, Hq_, d_)).to(cache_dtype)
    k_cache = torch.empty((pool, Hkv_, P, d_), dtype=cache_dtype, device=device)
    v_cache = torch.empty((pool, Hkv_, P, d_), dtype=cache_dtype, device=device)
    step = max(1, (1 << 27) // (Hkv_ * P * d_))
    for cache in (k_cache, v_cache):
        for p0 in range(0, pool, step):
            p1 = min(pool, p0 + step)
            cache[p0:p1] = normal((p1 - p0, Hkv_, P, d_)).to(cache_dtype)

    # 4. planted heavy hitters
    kind = shape.planted[0] if shape.planted else None
    nblk_of = [_ceil_div(x, shape.block_size) for x in lens]
    planted_pos = {}
    for b in range(Bn):
        Lb = lens[b]
        ws = Lb if shape.window <= 0 else max(0, Lb - shape.window)
        if ws <= 0 or kind is None:
            continue
        for h in range(Hkv_):
            if kind == "positions":
                cnt = min(int(shape.planted[1]), ws)
                pos = torch.randperm(ws, generator=cpu_gen)[:cnt]
            elif kind == "token_frac":
                cnt = min(int(round(shape.planted[1] * Lb)), ws)
                pos = torch.randperm(ws, generator=cpu_gen)[:cnt]
            elif kind == "block_clusters":
                frac, clusters = shape.planted[1], int(shape.planted[2])
                n_blk = max(1, int(round(frac * nblk_of[b])))
                per = max(1, n_blk // clusters)
                cand_blocks = _ceil_div(ws, shape.block_size)
                starts = []
                for _ in range(clusters):
                    hi_start = max(1, cand_blocks - per)
                    starts.append(int(torch.randint(0, hi_start, (1,), generator=cpu_gen)))
                blocks = sorted({s + i for s in starts for i in range(per) if s + i < cand_blocks})
                toks = [t for j in blocks
                        for t in range(j * shape.block_size,
                                       min((j + 1) * shape.block_size, ws))]
                pos = torch.tensor(toks, dtype=torch.int64)
            else:
                raise ValueError(f"unknown planting {kind}")
            if pos.numel() == 0:
                continue
            if is_verify[b]:
                rows = q_full[b, :, h * G:(h + 1) * G].float().reshape(-1, d_)
            else:
                rows = q_draft_own[b, 0, h * G:(h + 1) * G].float()
            qbar = rows.mean(dim=0)
            norm = float(qbar.norm())
            if norm == 0.0:
                continue
            lam = 4.0 * math.sqrt(d_) / norm
            add = (lam / norm) * qbar                      # lambda * u
            pos = pos.to(torch.int64)
            pages = table[b, (pos // P)].to(torch.int64).to(device)
            slots = (pos % P).to(device)
            kf = k_cache[pages, h, slots].float() + add.unsqueeze(0).to(device)
            k_cache[pages, h, slots] = kf.to(cache_dtype)
            planted_pos[(b, h)] = sorted(pos.tolist())

    # 5. sub-batches
    vids = [b for b in range(Bn) if is_verify[b]]
    if shape.p_verify is None:
        dids = list(range(Bn))
    else:
        dids = [b for b in range(Bn) if not is_verify[b]]
    budgets = [budget_for(shape, x) for x in lens]
    max_blocks = max(nblk_of)

    def sub(ids, q):
        ids_t = torch.tensor(ids, dtype=torch.int64)
        return Batch(
            q=q[ids_t.to(q.device)].contiguous() if ids else q[:0].contiguous(),
            page_table=table[ids_t].contiguous().to(device),
            seq_lens=torch.tensor([lens[b] for b in ids], dtype=torch.int32).to(device),
            budget=torch.tensor([budgets[b] for b in ids], dtype=torch.int32).to(device),
            req_ids=list(ids),
        )

    verify = sub(vids, q_full) if vids else None
    if shape.p_verify is None:
        # the draft query is the query of the last verify position, over the
        # same cache and length
        draft = sub(dids, q_full[:, shape.n_q - 1:shape.n_q])
    else:
        draft = sub(dids, q_draft_own) if dids else None
    max_sel = max(budgets)
    if draft is not None and shape.p_verify is not None:
        # given selection lists for draft-only requests
        sel = torch.full((draft.B, Hkv_, max_sel), -1, dtype=torch.int32)
        cnt = torch.zeros((draft.B, Hkv_), dtype=torch.int32)
        for i, b in enumerate(dids):
            Lb = lens[b]
            ws = Lb if shape.window <= 0 else max(0, Lb - shape.window)
            ncand = min(nblk_of[b], _ceil_div(ws, shape.block_size))
            n_eff = min(budgets[b], ncand, max_sel)
            for h in range(Hkv_):
                pick = torch.randperm(ncand, generator=cpu_gen)[:n_eff].sort().values
                sel[i, h, :n_eff] = pick.to(torch.int32)
                cnt[i, h] = n_eff
        draft.sel = sel.to(device)
        draft.sel_count = cnt.to(device)

    # 6. sparse verify layouts
    if verify is not None and shape.layout_shared is not None:
        rs = torch.full((verify.B, Hkv_, shape.n_q, max_sel), -1, dtype=torch.int32)
        rc = torch.zeros((verify.B, Hkv_, shape.n_q), dtype=torch.int32)
        for i, b in enumerate(vids):
            Lb = lens[b]
            ws = Lb if shape.window <= 0 else max(0, Lb - shape.window)
            ncand = min(nblk_of[b], _ceil_div(ws, shape.block_size))
            n_eff = min(budgets[b], ncand, max_sel)
            n_shared = int(round(shape.layout_shared * n_eff))
            for h in range(Hkv_):
                heavy = {t // shape.block_size for t in planted_pos.get((b, h), [])
                         if t // shape.block_size < ncand}
                order = torch.randperm(ncand, generator=cpu_gen).tolist()
                core = ([j for j in order if j in heavy] +
                        [j for j in order if j not in heavy])[:n_shared]
                core_set = set(core)
                rest = [j for j in order if j not in core_set]
                for qi in range(shape.n_q):
                    own = torch.randperm(len(rest), generator=cpu_gen)[:n_eff - n_shared]
                    pick = core + [rest[int(k)] for k in own]
                    shuf = torch.randperm(len(pick), generator=cpu_gen).tolist()
                    rs[i, h, qi, :len(pick)] = torch.tensor([pick[k] for k in shuf],
                                                            dtype=torch.int32)
                    rc[i, h, qi] = len(pick)
        verify.row_sel = rs.to(device)
        verify.row_sel_count = rc.to(device)

    return Workload(shape=shape, seed=seed, k_cache=k_cache, v_cache=v_cache,
                    seq_lens_all=lens, verify=verify, draft=draft,
                    sm_scale=1.0 / math.sqrt(d_), max_blocks=max_blocks, max_sel=max_sel,
                    extras={"planted": planted_pos, "is_verify": is_verify})


def to_numpy64(t: torch.Tensor):
    """Exact host copy in fp64 (bf16/fp32 -> fp64 is exact)."""
    return t.detach().to("cpu").to(torch.float64).numpy()
