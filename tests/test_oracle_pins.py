"""Pins of the fp64 oracle to things other than itself.

* verify O/LSE: torch's scaled_dot_product_attention and logsumexp in fp64 on
  the CPU with an explicit bottom-right causal mask (library routines);
* paged addressing: gather is the inverse of a scatter built from a
  contiguous cache;
* block scores: an explicit probability matrix from torch.softmax, the
  closed form of uniform attention (tests/golden/uniform_attention.json),
  and the row-mass invariant;
* Top-N: a rank-counting definition on brute force, fuzzed with ties, and
  hand-derived fixtures (tests/golden/topk_cases.json);
* draft: SDPA with the boolean mask of the token set; dense and sliding
  window as special cases;
* merge: partials of a partition computed by SDPA merge to the unsplit
  result; identity, associativity and the empty case;
* KV update: a write equals slicing the logical per-request sequence (built
  by torch indexing, not page arithmetic); out-of-range writes change
  nothing; after a commit, verify equals SDPA on the explicitly truncated
  sequence.

The mutation tests at the end plant plausible mistakes in copies of oracle
functions and check that the pins above reject them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import sss_oracle as so

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(1234)


def paged_case(B=2, Ls=(37, 64), Hq=4, Hkv=2, d=16, P=8, n_q=3, seed=0, sigma=1.0):
    g = np.random.default_rng(seed)
    Ls = list(Ls)[:B]
    npg = [-(-L // P) for L in Ls]
    pool = sum(npg)
    perm = g.permutation(pool)
    table = np.zeros((B, max(npg)), dtype=np.int32)
    off = 0
    for b in range(B):
        table[b, :npg[b]] = perm[off:off + npg[b]]
        off += npg[b]
    kc = g.normal(0, sigma, (pool, Hkv, P, d))
    vc = g.normal(0, sigma, (pool, Hkv, P, d))
    q = g.normal(0, sigma, (B, n_q, Hq, d))
    return q, kc, vc, table, np.array(Ls, dtype=np.int32)


def contiguous(kc, table, L, h):
    """Independent gather via torch indexing of the flattened token axis."""
    P = kc.shape[2]
    t = torch.arange(L)
    pages = torch.as_tensor(table)[t // P].long()
    return torch.as_tensor(kc)[pages, h, t % P]


# --------------------------------------------------------------------------
# verify
# --------------------------------------------------------------------------
def sdpa_verify(q, kc, vc, table, lens, scale):
    B, n_q, Hq, d = q.shape
    Hkv = kc.shape[1]
    G = Hq // Hkv
    O = np.zeros_like(q)
    LSE = np.zeros((B, n_q, Hq))
    for b in range(B):
        L = int(lens[b])
        for hq in range(Hq):
            h = hq // G
            K = contiguous(kc, table[b], L, h).double()
            V = contiguous(vc, table[b], L, h).double()
            Q = torch.as_tensor(q[b, :, hq]).double()
            pos = torch.arange(n_q) + L - n_q
            mask = torch.arange(L)[None, :] <= pos[:, None]
            out = F.scaled_dot_product_attention(Q[None], K[None], V[None], attn_mask=mask[None],
                                                 scale=scale)[0]
            logits = (Q @ K.T) * scale
            logits = logits.masked_fill(~mask, -math.inf)
            O[b, :, hq] = out.numpy()
            LSE[b, :, hq] = torch.logsumexp(logits, dim=-1).numpy()
    return O, LSE


def verify_err(verify_fn, **kw):
    q, kc, vc, table, lens = paged_case(**kw)
    scale = 1.0 / math.sqrt(q.shape[-1])
    O, LSE = verify_fn(q, kc, vc, table, lens, scale)
    Or, LSEr = sdpa_verify(q, kc, vc, table, lens, scale)
    return max(np.abs(O - Or).max(), np.abs(LSE - LSEr).max())


@pytest.mark.parametrize("kw", [
    dict(),                                         # GQA G=2, ragged lengths
    dict(Hq=4, Hkv=4, n_q=2),                       # MHA
    dict(Hq=8, Hkv=1, n_q=1, Ls=(5, 33)),           # MQA, single query = plain decode
    dict(n_q=5, Ls=(5, 19), P=4),                   # L == n_q (first row sees 1 token)
    dict(B=1, Ls=(130,), P=16, d=8, n_q=4, sigma=3.0),  # peaky softmax
])
def test_verify_matches_sdpa(kw):
    assert verify_err(oracle.verify, **kw) < 1e-12


def test_gather_inverts_scatter():
    g = np.random.default_rng(5)
    L, P, Hkv, d = 45, 8, 3, 4
    Kc = g.normal(size=(Hkv, L, d))
    npg = -(-L // P)
    perm = g.permutation(npg + 3)[:npg]
    kc = np.full((npg + 3, Hkv, P, d), np.nan)
    for t in range(L):
        kc[perm[t // P], :, t % P] = Kc[:, t]
    for h in range(Hkv):
        K, V = oracle.gather_unit(kc, kc, perm, L, h)
        assert np.array_equal(K, Kc[h]) and np.array_equal(V, Kc[h])


def test_causality_perturbation():
    q, kc, vc, table, lens = paged_case(B=1, Ls=(29,), n_q=4, P=4)
    scale = 0.3
    O0, L0 = oracle.verify(q, kc, vc, table, lens, scale)
    L = int(lens[0])
    for i in range(4):
        pos = L - 4 + i
        kc2, vc2 = kc.copy(), vc.copy()
        for t in range(pos + 1, L):
            pg = table[0, t // 4]
            kc2[pg, :, t % 4] += 5.0
            vc2[pg, :, t % 4] -= 3.0
        O1, L1 = oracle.verify(q, kc2, vc2, table, lens, scale)
        assert np.array_equal(O1[0, i], O0[0, i]) and np.array_equal(L1[0, i], L0[0, i])
        # and a change at a visible position does move the row
        pg = table[0, pos // 4]
        vc2[pg, :, pos % 4] += 1.0
        O2, _ = oracle.verify(q, kc2, vc2, table, lens, scale)
        assert np.abs(O2[0, i] - O0[0, i]).max() > 1e-3


# --------------------------------------------------------------------------
# block scores
# --------------------------------------------------------------------------
def softmax_block_scores(q, kc, vc, table, lens, scale, bs, max_blocks, r0):
    """Explicit probability matrix from torch.softmax, summed per block."""
    B, n_q, Hq, d = q.shape
    Hkv = kc.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hkv, max_blocks))
    for b in range(B):
        L = int(lens[b])
        pos = torch.arange(n_q) + L - n_q
        mask = torch.arange(L)[None, :] <= pos[:, None]
        for h in range(Hkv):
            K = contiguous(kc, table[b], L, h).double()
            tot = torch.zeros(L, dtype=torch.float64)
            for g in range(G):
                Q = torch.as_tensor(q[b, :, h * G + g]).double()
                Pm = torch.softmax(((Q @ K.T) * scale).masked_fill(~mask, -math.inf), dim=-1)
                tot += Pm[r0:].sum(0)
            nblk = -(-L // bs)
            padded = torch.zeros(nblk * bs, dtype=torch.float64)
            padded[:L] = tot
            out[b, h, :nblk] = padded.view(nblk, bs).sum(1).numpy()
    return out


@pytest.mark.parametrize("r0", [0, 1])
@pytest.mark.parametrize("bs", [4, 16])
def test_block_scores_match_softmax_matrix(r0, bs):
    q, kc, vc, table, lens = paged_case(B=2, Ls=(50, 64), P=4, n_q=3)
    scale = 0.25
    mb = 20
    _, _, S = oracle.verify_with_scores(q, kc, vc, table, lens, scale, bs, mb, r0)
    ref = softmax_block_scores(q, kc, vc, table, lens, scale, bs, mb, r0)
    assert np.abs(S - ref).max() < 1e-12
    # row-mass invariant: every scored row contributes exactly 1
    G = q.shape[2] // kc.shape[1]
    assert np.allclose(S.sum(-1), (3 - r0) * G, atol=1e-12, rtol=0)


def test_block_scores_uniform_closed_form():
    """Hand-derived fixture: with q = 0 every visible token gets 1/(pos+1)."""
    with open(os.path.join(GOLDEN, "uniform_attention.json")) as f:
        case = json.load(f)
    L, n_q, bs, d = case["L"], case["n_q"], case["block_size"], case["d"]
    q = np.zeros((1, n_q, 1, d))
    vals = np.arange(L * d, dtype=np.float64).reshape(L, d) / 7.0
    kc = np.random.default_rng(2).normal(size=(L, 1, 1, d))
    vc = vals.reshape(L, 1, 1, d)
    table = np.arange(L, dtype=np.int32)[None]
    O, LSE, S = oracle.verify_with_scores(q, kc, vc, table, np.array([L]), 1.0, bs,
                                           case["max_blocks"], 0)
    assert np.allclose(S[0, 0], case["block_scores"], atol=1e-14, rtol=0)
    assert np.allclose(LSE[0, :, 0], [math.log(p + 1) for p in case["positions"]], atol=1e-14)
    for i, p in enumerate(case["positions"]):
        assert np.allclose(O[0, i, 0], vals[:p + 1].mean(0), atol=1e-12)


def test_planted_blocks_carry_top_mass():
    """Sanity on the tiny fp32 workload: every planted position lies in one
    of the highest-scoring blocks."""
    from sparse_self_speculative_sss_amd import workload as W
    wl = W.make("tiny_fp32_b1_l512", seed=0)
    vb = wl.verify
    q = W.to_numpy64(vb.q)
    _, _, S = oracle.verify_with_scores(q, W.to_numpy64(wl.k_cache), W.to_numpy64(wl.v_cache),
                                        vb.page_table.numpy(), vb.seq_lens.numpy(), wl.sm_scale,
                                        16, wl.max_blocks, 0)
    planted_blocks = {p // 16 for p in wl.extras["planted"][(0, 0)]}
    top = set(np.argsort(-S[0, 0])[:len(planted_blocks)].tolist())
    assert planted_blocks == top


# --------------------------------------------------------------------------
# Top-N
# --------------------------------------------------------------------------
def rank_select(scores, L, bs, budget, window, max_sel):
    """Brute force by rank counting: j is kept iff fewer than N_eff
    candidates beat it (higher score, or equal score and lower index)."""
    ws = L if window <= 0 else max(0, L - window)
    nblk = -(-L // bs)
    C = [j for j in range(nblk) if j * bs < ws]
    n_eff = min(budget, len(C), max_sel)
    keep = []
    for j in C:
        beaten = sum(1 for i in C if scores[i] > scores[j] or (scores[i] == scores[j] and i < j))
        if beaten < n_eff:
            keep.append(j)
    return keep


def test_topk_bruteforce_fuzz():
    g = np.random.default_rng(99)
    for trial in range(400):
        bs = int(g.choice([1, 4, 16]))
        L = int(g.integers(1, 40 * bs))
        nblk = -(-L // bs)
        window = int(g.choice([0, 1, bs, 3 * bs + 1, 10 ** 6]))
        budget = int(g.integers(0, nblk + 3))
        max_sel = int(g.integers(1, nblk + 3))
        levels = int(g.choice([2, 3, 1000]))      # few levels force ties
        scores = (g.integers(0, levels, nblk + 5) / levels).astype(np.float32)
        got = oracle.topk_unit(scores, L, bs, budget, window, max_sel)
        assert got == rank_select(scores, L, bs, budget, window, max_sel), trial


def test_topk_golden_cases():
    with open(os.path.join(GOLDEN, "topk_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        got = oracle.topk_unit(np.array(c["scores"], dtype=np.float32), c["L"], c["block_size"],
                               c["budget"], c["window"], c["max_sel"])
        assert got == c["expected"], c["why"]


def test_topk_batch_padding():
    scores = np.array([[[0.1, 0.5, 0.5, 0.2, 0.9, 0.0]]], dtype=np.float32)
    sel, cnt = oracle.block_topk(scores, np.array([90]), 16, np.array([3]), 16, 5)
    # L=90, bs=16 -> 6 blocks; window 16 -> start 74; candidates j*16 < 74 -> 0..4
    assert cnt.tolist() == [[3]]
    assert sel.tolist() == [[[1, 2, 4, -1, -1]]]


# --------------------------------------------------------------------------
# draft
# --------------------------------------------------------------------------
def sdpa_draft(q, kc, vc, table, lens, sel, cnt, bs, window, scale):
    B, _, Hq, d = q.shape
    Hkv = kc.shape[1]
    G = Hq // Hkv
    O = np.zeros((B, 1, Hq, d))
    for b in range(B):
        L = int(lens[b])
        ws = L if window <= 0 else max(0, L - window)
        for hq in range(Hq):
            h = hq // G
            t = torch.arange(L)
            in_sel = torch.zeros(L, dtype=torch.bool)
            for j in sel[b, h, :cnt[b, h]]:
                in_sel |= (t // bs == int(j))
            mask = (in_sel & (t < ws)) | (t >= ws)
            K = contiguous(kc, table[b], L, h).double()
            V = contiguous(vc, table[b], L, h).double()
            Q = torch.as_tensor(q[b, 0, hq]).double()[None]
            O[b, 0, hq] = F.scaled_dot_product_attention(Q[None], K[None], V[None],
                                                         attn_mask=mask[None, None],
                                                         scale=scale)[0, 0].numpy()
    return O


def random_sel(g, lens, Hkv, bs, window, budget, max_sel):
    B = len(lens)
    sel = np.full((B, Hkv, max_sel), -1, dtype=np.int32)
    cnt = np.zeros((B, Hkv), dtype=np.int32)
    for b, L in enumerate(lens):
        ws = L if window <= 0 else max(0, L - window)
        C = [j for j in range(-(-L // bs)) if j * bs < ws]
        n = min(budget, len(C), max_sel)
        for h in range(Hkv):
            pick = sorted(g.choice(C, n, replace=False).tolist()) if n else []
            sel[b, h, :n] = pick
            cnt[b, h] = n
    return sel, cnt


@pytest.mark.parametrize("window", [0, 5, 16])
def test_draft_matches_masked_sdpa(window):
    g = np.random.default_rng(3)
    q, kc, vc, table, lens = paged_case(B=2, Ls=(53, 80), n_q=1, P=4)
    sel, cnt = random_sel(g, lens.tolist(), kc.shape[1], 8, window, 3, 4)
    O, _ = oracle.draft(q, kc, vc, table, lens, sel, cnt, 8, window, 0.4)
    ref = sdpa_draft(q, kc, vc, table, lens, sel, cnt, 8, window, 0.4)
    assert np.abs(O - ref).max() < 1e-12


def test_draft_full_budget_equals_dense_decode():
    q, kc, vc, table, lens = paged_case(B=2, Ls=(53, 80), n_q=1, P=4)
    nblk = -(-80 // 8)
    sel = np.tile(np.arange(nblk, dtype=np.int32), (2, 2, 1))
    cnt = np.array([[-(-53 // 8)] * 2, [nblk] * 2], dtype=np.int32)
    for window in (0, 7):
        O, LSE = oracle.draft(q, kc, vc, table, lens, sel, cnt, 8, window, 0.4)
        Od, LSEd = sdpa_verify(q, kc, vc, table, lens, 0.4)
        assert np.abs(O - Od).max() < 1e-12 and np.abs(LSE - LSEd).max() < 1e-12


def test_draft_window_only_is_sliding_window():
    q, kc, vc, table, lens = paged_case(B=1, Ls=(70,), n_q=1, P=4)
    W = 9
    sel = np.full((1, 2, 2), -1, dtype=np.int32)
    cnt = np.zeros((1, 2), dtype=np.int32)
    O, _ = oracle.draft(q, kc, vc, table, lens, sel, cnt, 8, W, 0.4)
    for hq in range(4):
        h = hq // 2
        K = contiguous(kc, table[0], 70, h).double()[70 - W:]
        V = contiguous(vc, table[0], 70, h).double()[70 - W:]
        Q = torch.as_tensor(q[0, 0, hq]).double()[None, None]
        ref = F.scaled_dot_product_attention(Q, K[None], V[None], scale=0.4)[0, 0]
        assert np.abs(O[0, 0, hq] - ref.numpy()).max() < 1e-12
    # window >= L is dense attention
    O2, _ = oracle.draft(q, kc, vc, table, lens, sel, cnt, 8, 1000, 0.4)
    Od, _ = sdpa_verify(q, kc, vc, table, lens, 0.4)
    assert np.abs(O2 - Od).max() < 1e-12


def test_draft_order_of_selection_irrelevant_and_empty_set():
    g = np.random.default_rng(8)
    q, kc, vc, table, lens = paged_case(B=1, Ls=(96,), n_q=1, P=8)
    sel = np.array([[[1, 4, 6, -1], [0, 2, 3, -1]]], dtype=np.int32)
    cnt = np.array([[3, 3]], dtype=np.int32)
    O1, L1 = oracle.draft(q, kc, vc, table, lens, sel, cnt, 8, 8, 0.4)
    O2, L2 = oracle.draft(q, kc, vc, table, lens, sel[:, :, [2, 0, 1, 3]], cnt, 8, 8, 0.4)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
    O3, L3 = oracle.draft(q, kc, vc, table, lens, sel, np.zeros_like(cnt), 8, 0, 0.4)
    assert np.all(O3 == 0) and np.all(np.isneginf(L3))


# --------------------------------------------------------------------------
# sparse verification: a layout per query position
# --------------------------------------------------------------------------
def sdpa_sparse_verify(q, kc, vc, table, lens, row_sel, row_cnt, bs, window, scale):
    """Masked SDPA: position i of (b, hq) sees its own selected blocks before
    the window start, the window, and nothing past L - n_q + i."""
    B, n_q, Hq, d = q.shape
    Hkv = kc.shape[1]
    G = Hq // Hkv
    O = np.zeros((B, n_q, Hq, d))
    LSE = np.zeros((B, n_q, Hq))
    for b in range(B):
        L = int(lens[b])
        ws = L if window <= 0 else max(0, L - window)
        t = torch.arange(L)
        for hq in range(Hq):
            h = hq // G
            mask = torch.zeros((n_q, L), dtype=torch.bool)
            for i in range(n_q):
                for j in row_sel[b, h, i, :max(0, int(row_cnt[b, h, i]))]:
                    mask[i] |= (t // bs == int(j)) & (t < ws)
                mask[i] |= t >= ws
                mask[i] &= t <= L - n_q + i
            K = contiguous(kc, table[b], L, h).double()
            V = contiguous(vc, table[b], L, h).double()
            Q = torch.as_tensor(q[b, :, hq]).double()
            live = mask.any(dim=1)
            out = F.scaled_dot_product_attention(Q[None], K[None], V[None],
                                                 attn_mask=mask[None], scale=scale)[0]
            logits = ((Q @ K.T) * scale).masked_fill(~mask, -math.inf)
            O[b, :, hq] = torch.where(live[:, None], out, torch.zeros_like(out)).numpy()
            LSE[b, :, hq] = torch.logsumexp(logits, dim=-1).numpy()
    return O, LSE


def random_row_sel(g, lens, Hkv, n_q, bs, window, budget, max_sel, shared):
    """Layouts with `shared` blocks common to every position of a unit and the
    rest drawn per position; entries shuffled, some repeated, -1 padded."""
    B = len(lens)
    sel = np.full((B, Hkv, n_q, max_sel), -1, dtype=np.int32)
    cnt = np.zeros((B, Hkv, n_q), dtype=np.int32)
    for b, L in enumerate(lens):
        ws = L if window <= 0 else max(0, L - window)
        C = [j for j in range(-(-L // bs)) if j * bs < ws]
        for h in range(Hkv):
            core = g.choice(C, min(shared, len(C)), replace=False).tolist() if C else []
            for i in range(n_q):
                extra = g.choice(C, min(budget, len(C)), replace=False).tolist() if C else []
                pick = (core + extra)[:max_sel]
                if pick and len(pick) < max_sel:
                    pick.append(pick[0])                       # a repeated entry
                g.shuffle(pick)
                sel[b, h, i, :len(pick)] = pick
                cnt[b, h, i] = len(pick)
    return sel, cnt


@pytest.mark.parametrize("window", [0, 2, 5, 16])
def test_sparse_verify_matches_masked_sdpa(window):
    g = np.random.default_rng(21)
    q, kc, vc, table, lens = paged_case(B=2, Ls=(53, 80), Hq=4, Hkv=2, n_q=4, P=4)
    sel, cnt = random_row_sel(g, lens.tolist(), 2, 4, 8, window, 2, 5, 1)
    O, LSE = oracle.sparse_verify(q, kc, vc, table, lens, sel, cnt, 8, window, 0.4)
    Or, LSEr = sdpa_sparse_verify(q, kc, vc, table, lens, sel, cnt, 8, window, 0.4)
    assert np.abs(O - Or).max() < 1e-12
    assert np.abs(LSE - LSEr).max() < 1e-12


def test_sparse_verify_full_layouts_equal_dense_verify():
    q, kc, vc, table, lens = paged_case(B=2, Ls=(53, 80), Hq=4, Hkv=2, n_q=3, P=4)
    nblk = -(-80 // 8)
    sel = np.tile(np.arange(nblk, dtype=np.int32), (2, 2, 3, 1))
    cnt = np.full((2, 2, 3), nblk, dtype=np.int32)
    Od, LSEd = sdpa_verify(q, kc, vc, table, lens, 0.4)
    for window in (0, 1, 7, 1000):
        O, LSE = oracle.sparse_verify(q, kc, vc, table, lens, sel, cnt, 8, window, 0.4)
        assert np.abs(O - Od).max() < 1e-12 and np.abs(LSE - LSEd).max() < 1e-12


def test_sparse_verify_single_position_equals_draft():
    g = np.random.default_rng(22)
    q, kc, vc, table, lens = paged_case(B=2, Ls=(53, 80), n_q=1, P=4)
    for window in (0, 5, 16):
        sel, cnt = random_sel(g, lens.tolist(), kc.shape[1], 8, window, 3, 4)
        O, LSE = oracle.sparse_verify(q, kc, vc, table, lens, sel[:, :, None], cnt[:, :, None],
                                      8, window, 0.4)
        Od, LSEd = oracle.draft(q, kc, vc, table, lens, sel, cnt, 8, window, 0.4)
        assert np.abs(O - Od).max() < 1e-12 and np.array_equal(np.isneginf(LSE), np.isneginf(LSEd))
        fin = np.isfinite(LSEd)
        assert np.abs(LSE[fin] - LSEd[fin]).max() < 1e-12


def test_sparse_verify_positions_independent_and_order_free():
    g = np.random.default_rng(23)
    q, kc, vc, table, lens = paged_case(B=1, Ls=(96,), Hq=4, Hkv=2, n_q=3, P=8)
    sel, cnt = random_row_sel(g, [96], 2, 3, 8, 8, 3, 6, 2)
    O1, L1 = oracle.sparse_verify(q, kc, vc, table, lens, sel, cnt, 8, 8, 0.4)
    # another position's layout does not move this one's output
    sel2, cnt2 = sel.copy(), cnt.copy()
    sel2[0, :, 2] = -1
    cnt2[0, :, 2] = 0
    O2, L2 = oracle.sparse_verify(q, kc, vc, table, lens, sel2, cnt2, 8, 8, 0.4)
    assert np.array_equal(O1[:, :2], O2[:, :2]) and np.array_equal(L1[:, :2], L2[:, :2])
    assert not np.allclose(O1[:, 2], O2[:, 2])
    # the order of a layout's entries is irrelevant
    perm = sel.copy()
    for i in range(3):
        for h in range(2):
            c = int(cnt[0, h, i])
            perm[0, h, i, :c] = perm[0, h, i, :c][::-1]
    O3, L3 = oracle.sparse_verify(q, kc, vc, table, lens, perm, cnt, 8, 8, 0.4)
    assert np.array_equal(O1, O3) and np.array_equal(L1, L3)
    # no selection and no window: empty sets apart from the causal window-free case
    O4, L4 = oracle.sparse_verify(q, kc, vc, table, lens, sel, np.zeros_like(cnt), 8, 0, 0.4)
    assert np.all(O4 == 0) and np.all(np.isneginf(L4))


def test_layout_union_contains_exactly_the_selected_blocks():
    g = np.random.default_rng(24)
    for window in (0, 8, 40):
        sel, cnt = random_row_sel(g, [96], 1, 4, 8, window, 3, 6, 2)
        ws = 96 if window == 0 else 96 - window
        u = oracle.layout_union(sel[0, 0], cnt[0, 0], 96, 8, window)
        assert u == sorted(set(u))
        picked = {int(j) for i in range(4) for j in sel[0, 0, i, :cnt[0, 0, i]] if j * 8 < ws}
        assert set(u) == picked
        # every query's token set lies inside the union's blocks plus the window
        for i in range(4):
            toks = oracle.sparse_verify_token_set(96, 4, i, sel[0, 0, i], cnt[0, 0, i], 8, window)
            assert all(t >= ws or t // 8 in picked for t in toks)


def _union_by_mask(row_sel, row_cnt, L, bs, window):
    """Independent construction: a boolean [positions][blocks] membership
    matrix from torch scatter, OR-reduced over positions, restricted to the
    blocks that start before the window start."""
    n_q, max_sel = row_sel.shape
    ws = L if window <= 0 else max(0, L - window)
    nblk = -(-L // bs)
    sel = torch.as_tensor(row_sel, dtype=torch.long)
    cnt = torch.as_tensor(row_cnt, dtype=torch.long).clamp(0, max_sel)
    slot_live = torch.arange(max_sel)[None, :] < cnt[:, None]          # entry within the count
    in_range = (sel >= 0) & (sel < nblk)
    member = torch.zeros((n_q, nblk + 1), dtype=torch.bool)
    idx = torch.where(slot_live & in_range, sel, torch.full_like(sel, nblk))  # dead -> spare column
    member.scatter_(1, idx, True)
    union = member[:, :nblk].any(0) & (torch.arange(nblk) * bs < ws)
    return torch.nonzero(union).flatten().tolist()


def test_layout_union_equals_boolean_mask_or():
    g = np.random.default_rng(31)
    for trial in range(300):
        n_q = int(g.integers(1, 9))
        bs = int(g.choice([1, 4, 16]))
        L = int(g.integers(1, 400))
        window = int(g.choice([0, 1, 7, 64, 1000]))
        max_sel = int(g.integers(1, 12))
        nblk = -(-L // bs)
        # entries: in range, duplicated, negative, past the request, in the window
        row_sel = g.integers(-3, nblk + 4, (n_q, max_sel)).astype(np.int32)
        if trial % 3 == 0:
            row_sel[:, -1] = row_sel[:, 0]
        row_cnt = g.integers(-2, max_sel + 3, n_q).astype(np.int32)   # clamped to [0, max_sel]
        got = oracle.layout_union(row_sel, row_cnt, L, bs, window)
        assert got == _union_by_mask(row_sel, row_cnt, L, bs, window), trial


def test_layout_union_pin_rejects_planted_mistakes():
    """A union that ignores the per-position counts, or keeps blocks inside
    the window, differs from the mask construction on these inputs."""
    row_sel = np.array([[2, 5, 3], [5, 8, -1]], dtype=np.int32)
    row_cnt = np.array([2, 3], dtype=np.int32)
    L, bs, window = 160, 16, 40          # window start 120: blocks 0..7 are candidates
    ref = _union_by_mask(row_sel, row_cnt, L, bs, window)
    assert ref == [2, 5]
    assert oracle.layout_union(row_sel, row_cnt, L, bs, window) == ref

    def ignore_counts(rs, rc, L_, bs_, w_):
        ws = L_ if w_ <= 0 else max(0, L_ - w_)
        return sorted({int(j) for j in rs.flatten() if j >= 0 and j * bs_ < ws})

    def keep_window(rs, rc, L_, bs_, w_):
        return sorted({int(j) for i in range(rs.shape[0]) for j in rs[i, :rc[i]]
                       if 0 <= j < -(-L_ // bs_)})

    assert ignore_counts(row_sel, row_cnt, L, bs, window) != ref     # picks up block 3
    assert keep_window(row_sel, row_cnt, L, bs, window) != ref       # keeps block 8


# --------------------------------------------------------------------------
# merge
# --------------------------------------------------------------------------
def test_merge_partition_equals_unsplit():
    g = np.random.default_rng(11)
    L, d, R = 77, 12, 6
    K = g.normal(size=(L, d))
    V = g.normal(size=(L, d))
    Q = g.normal(size=(R, d))
    pos = np.array([L - 1] * R)
    cuts = [0, 5, 6, 30, 77]
    parts = [oracle.attention_partial(Q, K, V, 0.3, pos, range(a, b)) for a, b in zip(cuts, cuts[1:])]
    O, LSE = oracle.merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    Qt, Kt, Vt = (torch.as_tensor(x) for x in (Q, K, V))
    ref = F.scaled_dot_product_attention(Qt[None], Kt[None], Vt[None], scale=0.3)[0]
    assert np.abs(O - ref.numpy()).max() < 1e-12
    assert np.abs(LSE - torch.logsumexp(Qt @ Kt.T * 0.3, -1).numpy()).max() < 1e-12
    # associativity
    a, b, c = parts[0], parts[1], parts[2]
    ab = oracle.merge(np.stack([a[0], b[0]]), np.stack([a[1], b[1]]))
    abc1 = oracle.merge(np.stack([ab[0], c[0]]), np.stack([ab[1], c[1]]))
    abc2 = oracle.merge(np.stack([a[0], b[0], c[0]]), np.stack([a[1], b[1], c[1]]))
    assert np.abs(abc1[0] - abc2[0]).max() < 1e-12 and np.abs(abc1[1] - abc2[1]).max() < 1e-12


def test_merge_identity_and_empty():
    g = np.random.default_rng(12)
    o = g.normal(size=(1, 4, 8))
    l = g.normal(size=(1, 4))
    O, LSE = oracle.merge(o, l)
    assert np.array_equal(O, o[0]) and np.array_equal(LSE, l[0])
    O, LSE = oracle.merge(g.normal(size=(3, 2, 8)), np.full((3, 2), -np.inf))
    assert np.all(O == 0) and np.all(np.isneginf(LSE))
    # an empty partial next to a live one carries no weight
    o2 = np.concatenate([o, g.normal(size=(1, 4, 8))])
    l2 = np.concatenate([l, np.full((1, 4), -np.inf)])
    O, LSE = oracle.merge(o2, l2)
    assert np.allclose(O, o[0], atol=1e-15) and np.allclose(LSE, l[0], atol=1e-15)


# --------------------------------------------------------------------------
# mutation tests: plant a mistake in a copy of the oracle, the pins must fail
# --------------------------------------------------------------------------
def _mut_verify_off_by_one(q, kc, vc, table, lens, scale):
    B, n_q, Hq, d = q.shape
    Hkv = kc.shape[1]
    G = Hq // Hkv
    O = np.zeros_like(q)
    LSE = np.zeros((B, n_q, Hq))
    for b in range(B):
        L = int(lens[b])
        for h in range(Hkv):
            K, V = oracle.gather_unit(kc, vc, table[b], L, h)
            qq = q[b, :, h * G:(h + 1) * G].reshape(n_q * G, -1)
            S = scale * (qq @ K.T)
            for i in range(n_q):
                S[i * G:(i + 1) * G, L - n_q + i:] = -np.inf   # drops the diagonal
            lse, P = so._softmax_rows(S)
            O[b, :, h * G:(h + 1) * G] = (P @ V).reshape(n_q, G, d)
            LSE[b, :, h * G:(h + 1) * G] = lse.reshape(n_q, G)
    return O, LSE


def _mut_verify_head_map(q, kc, vc, table, lens, scale):
    B, n_q, Hq, d = q.shape
    Hkv = kc.shape[1]
    O = np.zeros_like(q)
    LSE = np.zeros((B, n_q, Hq))
    for b in range(B):
        L = int(lens[b])
        for hq in range(Hq):
            K, V = oracle.gather_unit(kc, vc, table[b], L, hq % Hkv)  # wrong GQA map
            o, lse, _ = oracle.verify_unit(q[b, :, hq:hq + 1], K, V, L, n_q, 1, scale)
            O[b, :, hq] = o
            LSE[b, :, hq] = lse
    return O, LSE


def _logical(kc, table, L, Hkv):
    """[L][Hkv][d] view of one request through torch indexing."""
    return torch.stack([contiguous(kc, table, L, h) for h in range(Hkv)], dim=1).numpy()


def test_kv_write_equals_logical_slice_assignment():
    g = np.random.default_rng(17)
    B, Hkv, d, P, n_new = 3, 2, 8, 4, 5
    q, kc, vc, table, lens = paged_case(B=B, Ls=(37, 20, 29), Hkv=Hkv, d=d, P=P, seed=4)
    pos0 = np.array([32, 15, 24], dtype=np.int32)      # the last n_new positions
    k_new = g.normal(size=(B, n_new, Hkv, d))
    v_new = g.normal(size=(B, n_new, Hkv, d))
    k2, v2 = oracle.kv_write(kc, vc, table, k_new, v_new, pos0)
    for b in range(B):
        L = int(lens[b])
        want_k = _logical(kc, table[b], L, Hkv)
        want_v = _logical(vc, table[b], L, Hkv)
        want_k[pos0[b]:pos0[b] + n_new] = k_new[b]
        want_v[pos0[b]:pos0[b] + n_new] = v_new[b]
        assert np.array_equal(_logical(k2, table[b], L, Hkv), want_k)
        assert np.array_equal(_logical(v2, table[b], L, Hkv), want_v)
    # pages no request uses are untouched
    used = {int(x) for b in range(B) for x in table[b, :-(-int(lens[b]) // P)]}
    for pg in range(kc.shape[0]):
        if pg not in used:
            assert np.array_equal(k2[pg], kc[pg])


def test_kv_write_out_of_range_and_identity():
    g = np.random.default_rng(18)
    q, kc, vc, table, lens = paged_case(B=2, Ls=(16, 16), P=4, seed=5)
    Hkv, d = kc.shape[1], kc.shape[3]
    bad_table = table.copy()
    bad_table[1, 1] = 10 ** 6                     # page id outside the pool
    k_new = g.normal(size=(2, 3, Hkv, d))
    pos0 = np.array([-3, 4], dtype=np.int32)      # request 0 entirely before 0
    k2, v2 = oracle.kv_write(kc, vc, bad_table, k_new, k_new, pos0)
    assert np.array_equal(k2, kc) and np.array_equal(v2, vc)
    far = np.array([4 * table.shape[1], 4 * table.shape[1] + 7], dtype=np.int32)
    k3, _ = oracle.kv_write(kc, vc, table, k_new, k_new, far)
    assert np.array_equal(k3, kc)
    # writing back what is there changes nothing
    cur = np.stack([_logical(kc, table[b], 16, Hkv)[5:8] for b in range(2)])
    k4, _ = oracle.kv_write(kc, vc, table, cur, cur, np.array([5, 5], dtype=np.int32))
    assert np.array_equal(k4, kc)


def test_kv_commit_closed_forms():
    lens = np.array([40, 17, 5, 9], dtype=np.int32)
    assert np.array_equal(oracle.kv_commit(lens, [5, 5, 5, 5], 5), lens)
    assert np.array_equal(oracle.kv_commit(lens, [0, 0, 0, 0], 5), lens - 5)
    assert np.array_equal(oracle.kv_commit(lens, [9, -2, 3, 1], 5), [40, 12, 3, 5])


def test_verify_after_commit_equals_truncated_sdpa():
    """Rolled-back positions are never read: verify on the committed length
    equals SDPA over the explicitly truncated logical sequence."""
    g = np.random.default_rng(19)
    n_q, Hkv, Hq, d, P = 4, 2, 4, 8, 4
    # pages allocated for 8 more tokens than the current lengths
    q, kc, vc, table, alloc = paged_case(B=2, Ls=(41, 34), Hq=Hq, Hkv=Hkv, d=d, P=P, n_q=n_q,
                                         seed=6)
    lens = alloc - 8
    keep = np.array([2, 4], dtype=np.int32)
    new_lens = oracle.kv_commit(lens, keep, n_q)
    # the next step's verify: n_q fresh positions on top of the kept prefix
    pos0 = new_lens.copy()
    k_new = g.normal(size=(2, n_q, Hkv, d))
    v_new = g.normal(size=(2, n_q, Hkv, d))
    k2, v2 = oracle.kv_write(kc, vc, table, k_new, v_new, pos0)
    L2 = new_lens + n_q
    O, LSE = oracle.verify(q, k2, v2, table, L2, 0.37)
    G = Hq // Hkv
    for b in range(2):
        L = int(L2[b])
        K = np.concatenate([_logical(kc, table[b], int(new_lens[b]), Hkv), k_new[b]])
        V = np.concatenate([_logical(vc, table[b], int(new_lens[b]), Hkv), v_new[b]])
        for hq in range(Hq):
            h = hq // G
            qt = torch.as_tensor(q[b, :, hq])[None, None]
            kt = torch.as_tensor(K[:, h])[None, None]
            vt = torch.as_tensor(V[:, h])[None, None]
            mask = torch.ones(n_q, L, dtype=torch.bool).tril(L - n_q)
            ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=0.37)[0, 0]
            s_ = (qt[0, 0] @ kt[0, 0].T) * 0.37
            lse = torch.logsumexp(s_.masked_fill(~mask, -math.inf), dim=-1)
            assert np.abs(O[b, :, hq] - ref.numpy()).max() < 1e-12
            assert np.abs(LSE[b, :, hq] - lse.numpy()).max() < 1e-12


def test_mutations_are_caught():
    assert verify_err(_mut_verify_off_by_one) > 1e-3
    assert verify_err(_mut_verify_head_map, Hq=4, Hkv=2) > 1e-3

    # Top-N with reversed tie-break must disagree with the rank definition
    def mut_topk(scores, L, bs, budget, window, max_sel):
        ws = L if window <= 0 else max(0, L - window)
        C = [j for j in range(-(-L // bs)) if j * bs < ws]
        ranked = sorted(C, key=lambda j: (-float(scores[j]), -j))
        return sorted(ranked[:min(budget, len(C), max_sel)])
    s = np.array([0.5, 0.5, 0.5, 0.1], dtype=np.float32)
    assert mut_topk(s, 64, 16, 2, 0, 4) != rank_select(s, 64, 16, 2, 0, 4)

    # block scores that forget the causal mask break the row-mass invariant
    q, kc, vc, table, lens = paged_case(B=1, Ls=(40,), P=4, n_q=3)
    K, V = oracle.gather_unit(kc, vc, table[0], 40, 0)
    qq = q[0, :, 0:2].reshape(6, -1)
    lse, P = so._softmax_rows(0.25 * (qq @ K.T))      # no mask
    bad = oracle.block_mass_unit(P, 40, 3, 2, 4, 0, 10)
    ref = softmax_block_scores(q, kc, vc, table, lens, 0.25, 4, 10, 0)[0, 0]
    assert np.abs(bad - ref).max() > 1e-3


def test_sparse_verify_mutations_are_caught():
    """Two plausible mistakes of a grouped execution fail the masked-SDPA pin:
    every query attending to the whole union of the group's layouts, and
    selected tokens escaping the causal limit when the window is shorter than
    the step."""
    g = np.random.default_rng(25)
    q, kc, vc, table, lens = paged_case(B=1, Ls=(80,), Hq=4, Hkv=2, n_q=4, P=4)
    sel, cnt = random_row_sel(g, [80], 2, 4, 8, 2, 2, 5, 1)
    ref, _ = sdpa_sparse_verify(q, kc, vc, table, lens, sel, cnt, 8, 2, 0.4)

    def mut_union(q_, kc_, vc_, table_, lens_, sel_, cnt_, bs, window, scale):
        u = np.full(sel_.shape[:3] + (64,), -1, dtype=np.int32)
        c = np.zeros_like(cnt_)
        for h in range(sel_.shape[1]):
            blocks = oracle.layout_union(sel_[0, h], cnt_[0, h], int(lens_[0]), bs, window)
            u[0, h, :, :len(blocks)] = blocks
            c[0, h, :] = len(blocks)
        return oracle.sparse_verify(q_, kc_, vc_, table_, lens_, u, c, bs, window, scale)

    def mut_causal(q_, kc_, vc_, table_, lens_, sel_, cnt_, bs, window, scale):
        B, n_q, Hq, d = q_.shape
        O = np.zeros((B, n_q, Hq, d))
        G = Hq // kc_.shape[1]
        L = int(lens_[0])
        for hq in range(Hq):
            K, V = oracle.gather_unit(kc_, vc_, table_[0], L, hq // G)
            for i in range(n_q):
                toks = oracle.draft_token_set(L, sel_[0, hq // G, i], int(cnt_[0, hq // G, i]),
                                              bs, window)
                S = scale * (q_[0, i, hq] @ K[toks].T)
                S[np.asarray(toks) > L - 1] = -np.inf              # limit of the last row
                lse, P = so._softmax_rows(S[None])
                O[0, i, hq] = (P @ V[toks])[0]
        return O, None

    assert np.abs(mut_union(q, kc, vc, table, lens, sel, cnt, 8, 2, 0.4)[0] - ref).max() > 1e-3
    assert np.abs(mut_causal(q, kc, vc, table, lens, sel, cnt, 8, 2, 0.4)[0] - ref).max() > 1e-3


def test_kv_write_mutation_is_caught():
    """An off-by-one write position, or a write into the wrong KV head, fails
    the logical-slice pin."""
    g = np.random.default_rng(20)
    q, kc, vc, table, lens = paged_case(B=1, Ls=(30,), Hkv=2, P=4, seed=7)
    Hkv, d = kc.shape[1], kc.shape[3]
    k_new = g.normal(size=(1, 3, Hkv, d))
    pos0 = np.array([27], dtype=np.int32)

    def mut_shift(kc_, vc_, table_, kn, vn, p0):
        return oracle.kv_write(kc_, vc_, table_, kn, vn, np.asarray(p0) + 1)

    def mut_heads(kc_, vc_, table_, kn, vn, p0):
        return oracle.kv_write(kc_, vc_, table_, kn[:, :, ::-1], vn[:, :, ::-1], p0)

    want = _logical(kc, table[0], 30, Hkv)
    want[27:30] = k_new[0]
    for fn in (mut_shift, mut_heads):
        k2, _ = fn(kc, vc, table, k_new, k_new, pos0)
        assert not np.array_equal(_logical(k2, table[0], 30, Hkv), want)
    k2, _ = oracle.kv_write(kc, vc, table, k_new, k_new, pos0)
    assert np.array_equal(_logical(k2, table[0], 30, Hkv), want)
