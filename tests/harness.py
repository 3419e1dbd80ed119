"""Shared test plumbing: run the HIP path through the binding, run the oracle
on the same seeded inputs (optionally on a sample of units), compare.

Test infrastructure only (it imports the oracle)."""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
from sparse_self_speculative_sss_amd import workload as W

# Tolerances against the fp64 oracle (bf16 in, fp32 accumulate)
O_MAX_ABS = 2e-2
O_MEAN_ABS = 2e-3
SCORE_ABS = 1e-3
# diagnostics: natural-log LSE and relative L2 of O
LSE_ABS = 1e-3
O_REL_L2 = 1e-2


def sss():
    from sparse_self_speculative_sss_amd import sss as mod
    return mod


def kv_of(wl: W.Workload, batch: W.Batch):
    return sss().paged_kv(wl.k_cache, wl.v_cache, batch.page_table, batch.seq_lens,
                          batch.max_seq_len)


# --------------------------------------------------------------------------
# HIP path
# --------------------------------------------------------------------------
def gpu_verify(wl, batch, num_splits=None, score_row_start=0, poison=True):
    dev = batch.q.device
    B, n_q, hq, d = batch.q.shape
    hkv = wl.k_cache.shape[1]
    mb = wl.max_blocks
    o = torch.empty_like(batch.q)
    lse = torch.empty((B, n_q, hq), dtype=torch.float32, device=dev)
    sc = torch.empty((B, hkv, mb), dtype=torch.float32, device=dev)
    if poison:
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        sc.fill_(float("nan"))
    ns = wl.shape.num_splits if num_splits is None else num_splits
    sss().verify_attn(kv_of(wl, batch), batch.q, wl.sm_scale, wl.shape.block_size, mb, o, lse, sc,
                      score_row_start=score_row_start, num_splits=ns)
    return o, lse, sc


def gpu_topk(wl, batch, scores, budget=None, window=None, max_sel=None):
    dev = scores.device
    B, hkv, _ = scores.shape
    ms = wl.max_sel if max_sel is None else max_sel
    sel = torch.full((B, hkv, ms), 12345, dtype=torch.int32, device=dev)
    cnt = torch.full((B, hkv), -7, dtype=torch.int32, device=dev)
    bud = batch.budget if budget is None else budget
    win = wl.shape.window if window is None else window
    sss().block_topk(scores, batch.seq_lens, wl.shape.block_size, bud, win, sel, cnt)
    return sel, cnt


def gpu_draft(wl, batch, sel, cnt, num_splits=0, window=None, poison=True):
    dev = batch.q.device
    o = torch.empty_like(batch.q)
    B, _, hq, _ = batch.q.shape
    lse = torch.empty((B, 1, hq), dtype=torch.float32, device=dev)
    if poison:
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
    win = wl.shape.window if window is None else window
    sss().draft_attn(kv_of(wl, batch), batch.q, wl.sm_scale, wl.shape.block_size, sel, cnt, win,
                     o, lse, num_splits=num_splits)
    return o, lse


def gpu_sparse_verify(wl, batch, row_sel, row_cnt, num_splits=0, window=None, poison=True):
    dev = batch.q.device
    B, n_q, hq, d = batch.q.shape
    o = torch.empty_like(batch.q)
    lse = torch.empty((B, n_q, hq), dtype=torch.float32, device=dev)
    if poison:
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
    win = wl.shape.window if window is None else window
    sss().sparse_verify_attn(kv_of(wl, batch), batch.q, wl.sm_scale, wl.shape.block_size,
                             row_sel, row_cnt, win, o, lse, num_splits=num_splits)
    return o, lse


# --------------------------------------------------------------------------
# oracle on a subset of requests: copy only those requests' pages
# --------------------------------------------------------------------------
def request_view(wl, batch, b):
    """Host fp64 copy of request b's pages (all KV heads) with its page table
    remapped to the copy.  Pure data movement; no attention arithmetic."""
    P = wl.shape.page_size
    L = int(batch.seq_lens[b])
    n = -(-L // P)
    pages = batch.page_table[b, :n].long()
    k = W.to_numpy64(wl.k_cache[pages.to(wl.k_cache.device)])
    v = W.to_numpy64(wl.v_cache[pages.to(wl.v_cache.device)])
    table = np.arange(n, dtype=np.int32)[None]
    return k, v, table, L


def oracle_verify_units(wl, batch, units, score_row_start=0):
    """Oracle O/LSE/scores for (b, h) units; returns dict unit -> arrays."""
    q = W.to_numpy64(batch.q)
    out = {}
    by_req = {}
    for b, h in units:
        by_req.setdefault(b, []).append(h)
    for b, hs in by_req.items():
        k, v, table, L = request_view(wl, batch, b)
        O, LSE, S = oracle.verify_with_scores(q[b:b + 1], k, v, table, np.array([L]), wl.sm_scale,
                                              wl.shape.block_size, wl.max_blocks, score_row_start,
                                              units=[(0, h) for h in hs])
        for h in hs:
            out[(b, h)] = (O[0], LSE[0], S[0, h])
    return out


def oracle_draft_units(wl, batch, sel, cnt, units, window=None):
    q = W.to_numpy64(batch.q)
    win = wl.shape.window if window is None else window
    out = {}
    by_req = {}
    for b, h in units:
        by_req.setdefault(b, []).append(h)
    for b, hs in by_req.items():
        k, v, table, L = request_view(wl, batch, b)
        O, LSE = oracle.draft(q[b:b + 1], k, v, table, np.array([L]), sel[b:b + 1], cnt[b:b + 1],
                              wl.shape.block_size, win, wl.sm_scale, units=[(0, h) for h in hs])
        for h in hs:
            out[(b, h)] = (O[0], LSE[0])
    return out


def oracle_sparse_units(wl, batch, row_sel, row_cnt, units, window=None):
    q = W.to_numpy64(batch.q)
    win = wl.shape.window if window is None else window
    out = {}
    by_req = {}
    for b, h in units:
        by_req.setdefault(b, []).append(h)
    for b, hs in by_req.items():
        k, v, table, L = request_view(wl, batch, b)
        O, LSE = oracle.sparse_verify(q[b:b + 1], k, v, table, np.array([L]), row_sel[b:b + 1],
                                      row_cnt[b:b + 1], wl.shape.block_size, win, wl.sm_scale,
                                      units=[(0, h) for h in hs])
        for h in hs:
            out[(b, h)] = (O[0], LSE[0])
    return out


def group_slice(wl, h):
    G = wl.shape.Hq // wl.shape.Hkv
    return slice(h * G, (h + 1) * G)


# --------------------------------------------------------------------------
# comparisons
# --------------------------------------------------------------------------
class Stats:
    def __init__(self):
        self.o_max = 0.0
        self.o_sum = 0.0
        self.o_n = 0
        self.lse_max = 0.0
        self.sc_max = 0.0
        self.rel_num = 0.0
        self.rel_den = 0.0

    def add_o(self, got, ref):
        diff = np.abs(got - ref)
        assert np.all(np.isfinite(got)), "non-finite O from the HIP path"
        self.o_max = max(self.o_max, float(diff.max()))
        self.o_sum += float(diff.sum())
        self.o_n += diff.size
        self.rel_num += float((diff ** 2).sum())
        self.rel_den += float((ref ** 2).sum())

    def add_lse(self, got, ref):
        fin = np.isfinite(ref)
        assert np.array_equal(np.isfinite(got), fin), "LSE finiteness differs"
        assert np.array_equal(got[~fin], ref[~fin])
        if fin.any():
            self.lse_max = max(self.lse_max, float(np.abs(got[fin] - ref[fin]).max()))

    def add_scores(self, got, ref):
        assert np.all(np.isfinite(got)), "non-finite block score"
        self.sc_max = max(self.sc_max, float(np.abs(got - ref).max()))

    @property
    def o_mean(self):
        return self.o_sum / max(1, self.o_n)

    @property
    def rel_l2(self):
        return math.sqrt(self.rel_num / self.rel_den) if self.rel_den > 0 else 0.0

    def check(self, what=""):
        msg = (f"{what}: O max {self.o_max:.3e} mean {self.o_mean:.3e} relL2 {self.rel_l2:.3e} "
               f"LSE max {self.lse_max:.3e} scores max {self.sc_max:.3e}")
        print(msg, flush=True)
        assert self.o_max <= O_MAX_ABS, msg
        assert self.o_mean <= O_MEAN_ABS, msg
        assert self.sc_max <= SCORE_ABS, msg
        assert self.lse_max <= LSE_ABS, msg
        assert self.rel_l2 <= O_REL_L2, msg
        return msg


def compare_verify(wl, batch, gpu_out, units, score_row_start=0, stats=None):
    o, lse, sc = (t.float().cpu().numpy() for t in gpu_out)
    st = stats or Stats()
    ref = oracle_verify_units(wl, batch, units, score_row_start)
    for (b, h), (Or, LSEr, Sr) in ref.items():
        gs = group_slice(wl, h)
        st.add_o(o[b, :, gs].astype(np.float64), Or[:, gs])
        st.add_lse(lse[b, :, gs].astype(np.float64), LSEr[:, gs])
        st.add_scores(sc[b, h].astype(np.float64), Sr)
    return st


def compare_draft(wl, batch, gpu_out, sel_np, cnt_np, units, window=None, stats=None):
    o, lse = (t.float().cpu().numpy() for t in gpu_out)
    st = stats or Stats()
    ref = oracle_draft_units(wl, batch, sel_np, cnt_np, units, window)
    for (b, h), (Or, LSEr) in ref.items():
        gs = group_slice(wl, h)
        if np.all(np.isneginf(LSEr[:, gs])):
            assert np.all(o[b, :, gs] == 0) and np.all(np.isneginf(lse[b, :, gs]))
            continue
        st.add_o(o[b, :, gs].astype(np.float64), Or[:, gs])
        st.add_lse(lse[b, :, gs].astype(np.float64), LSEr[:, gs])
    return st


def compare_sparse(wl, batch, gpu_out, row_sel_np, row_cnt_np, units, window=None, stats=None):
    """Rows with an empty token set must be exactly O = 0, LSE = -inf (the
    LSE comparison checks the infinities, the O comparison the zeros)."""
    o, lse = (t.float().cpu().numpy() for t in gpu_out)
    st = stats or Stats()
    ref = oracle_sparse_units(wl, batch, row_sel_np, row_cnt_np, units, window)
    for (b, h), (Or, LSEr) in ref.items():
        gs = group_slice(wl, h)
        st.add_o(o[b, :, gs].astype(np.float64), Or[:, gs])
        st.add_lse(lse[b, :, gs].astype(np.float64), LSEr[:, gs])
        empty = np.isneginf(LSEr[:, gs])
        assert np.all(o[b, :, gs][empty] == 0)
    return st


def all_units(batch, hkv):
    return [(b, h) for b in range(batch.B) for h in range(hkv)]


def sample_units(batch, hkv, n, seed=0):
    g = np.random.default_rng(seed)
    allu = all_units(batch, hkv)
    if n >= len(allu):
        return allu
    idx = g.choice(len(allu), n, replace=False)
    return [allu[i] for i in sorted(idx)]


def oracle_selection(wl, batch, units, score_row_start=0):
    """Oracle scores (rounded to fp32) and oracle Top-N for the given units;
    rows of units not listed stay zero / -1."""
    B = batch.B
    hkv = wl.k_cache.shape[1]
    ref = oracle_verify_units(wl, batch, units, score_row_start)
    scores = np.zeros((B, hkv, wl.max_blocks), dtype=np.float32)
    for (b, h), (_, _, S) in ref.items():
        scores[b, h] = S.astype(np.float32)
    sel, cnt = oracle.block_topk(scores, batch.seq_lens.cpu().numpy(), wl.shape.block_size,
                                 batch.budget.cpu().numpy(), wl.shape.window, wl.max_sel)
    return scores, sel, cnt
