"""Plain fp64 CPU oracle for sparse self-speculative decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the test suite, the smoke check and the CPU-baseline
leg of the benchmark use it.  It shares no code with the HIP library.

What it computes (the pages it follows):

* SparseSpec -- "Accelerating Large-Scale Reasoning Model Inference:
  Self-Speculative Decoding with Sparse Attention", §4.1 (PillarAttn) and
  Fig. 7: a verification step runs full attention over the whole KV cache;
  the attention scores it produces are dumped (logits plus log-sum-exp), the
  scores of the draft tokens and of the query heads of one GQA group are
  aggregated, and a Top-K over the aggregate gives the sparse pattern that the
  next k draft steps use.  §4.2: KV lives in a paged cache (PagedAttention).
* SpecAttn -- "SpecAttn: Co-Designing Sparse Attention with Self-Speculative
  Decoding", 方法详解 (technical framework): the critical KV entries are a
  by-product of verification and drafting loads only those entries.

* SpecSA -- "SpecSA：融合推测解码与稀疏注意力的高效LLM推理框架", 核心创新 /
  刷新/复用NSA内核融合 (refresh / reuse): the KV of accepted speculative
  tokens is kept for later queries, the KV of rejected ones is refreshed.
  Here: writing the new positions' K/V into the paged cache (kv_write) and
  shortening each request to the positions it keeps (kv_commit).
  核心创新 / 重叠感知分组查询执行 (overlap-aware grouped query execution) and
  稀疏布局的动态管理 (sparse layout management): each query position of a
  verify step has its own sparse layout (sparse_verify); a grouped execution
  loads the union of the layouts once (layout_union).

Every step below is the plain mathematical definition written out with numpy
(matrix products, exp/log, Python sorting).  No blocking, online softmax,
splitting or fusion is used anywhere here.

Readings taken where the pages are silent:

* Causal alignment: ``seq_lens[b]`` counts every KV token of request b,
  including the n_q new query tokens, which sit at the tail; verify row i sits
  at position ``L - n_q + i`` and sees tokens ``t <= L - n_q + i``.
* The block score is the softmax probability mass summed (not averaged) over
  the scored rows; a positive rescale does not change the Top-N order.
* Rows are ordered ``r = i * G + g`` for query position i and group head g;
  ``score_row_start`` skips the first query positions (1 scores only the k
  draft tokens, 0 also scores the bonus row).
* Natural-log LSE; scale passed explicitly.
* Top-N candidates are the blocks that start before the recent window; ties
  go to the lower block index; output ascending, padded with -1.
* The draft attends to the tokens of the selected blocks that lie before the
  window start, plus every token of the window.
* An empty attention set yields O = 0 and LSE = -inf.

Parity pins for each function live in tests/test_oracle_pins.py.
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = -math.inf


def _f64(x) -> np.ndarray:
    """Exact widening to fp64 (bf16 and fp32 values are representable)."""
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# Paged KV addressing (SparseSpec §4.2: PagedAttention-style paged cache)
# ---------------------------------------------------------------------------
def gather_unit(k_cache, v_cache, page_table_row, seq_len: int, kv_head: int):
    """Return the contiguous K and V rows [L][d] (fp64) of one request/KV head.

    Cache layout: ``[num_pages][num_kv_heads][page_size][head_dim]``; token t
    of the request lives in page ``page_table_row[t // page_size]`` at slot
    ``t % page_size``.
    """
    page_size = k_cache.shape[2]
    d = k_cache.shape[3]
    K = np.empty((seq_len, d), dtype=np.float64)
    V = np.empty((seq_len, d), dtype=np.float64)
    n_pages = (seq_len + page_size - 1) // page_size
    for p in range(n_pages):
        page = int(page_table_row[p])
        lo = p * page_size
        hi = min(lo + page_size, seq_len)
        K[lo:hi] = k_cache[page, kv_head, : hi - lo]
        V[lo:hi] = v_cache[page, kv_head, : hi - lo]
    return K, V


def _softmax_rows(S: np.ndarray):
    """Row-wise natural-log LSE and probabilities of a logit matrix that may
    hold -inf entries.  A row with no finite entry gives LSE -inf, p = 0."""
    lse = np.full(S.shape[0], NEG_INF)
    P = np.zeros_like(S)
    for r in range(S.shape[0]):
        row = S[r]
        finite = np.isfinite(row)
        if not finite.any():
            continue
        m = row[finite].max()
        total = np.exp(row[finite] - m).sum()
        lse[r] = m + math.log(total)
        P[r, finite] = np.exp(row[finite] - lse[r])
    return lse, P


# ---------------------------------------------------------------------------
# Verify attention + per-block importance (SparseSpec §4.1, Fig. 7;
# SpecAttn 方法详解)
# ---------------------------------------------------------------------------
def verify_unit(q_rows, K, V, seq_len: int, n_q: int, group: int, sm_scale: float):
    """Dense causal attention of the R = n_q * group rows of one (request,
    KV head) unit over its whole KV.

    ``q_rows`` is [n_q][group][d]; row r = i * group + g.  Returns
    (O [R][d], LSE [R], P [R][L]) in fp64, P being the exact softmax
    probabilities (zero where masked).
    """
    q = _f64(q_rows).reshape(n_q * group, -1)
    S = sm_scale * (q @ K.T)                      # [R][L] logits
    for i in range(n_q):
        pos = seq_len - n_q + i                   # bottom-right causal alignment
        S[i * group:(i + 1) * group, pos + 1:] = NEG_INF
    lse, P = _softmax_rows(S)
    O = P @ V
    return O, lse, P


def verify(q, k_cache, v_cache, page_table, seq_lens, sm_scale: float):
    """Verify attention for a batch.

    q: [B][n_q][Hq][d]; returns O [B][n_q][Hq][d] and LSE [B][n_q][Hq] (fp64).
    Query head hq reads KV head hq // G.
    """
    B, n_q, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    O = np.zeros((B, n_q, Hq, d))
    LSE = np.zeros((B, n_q, Hq))
    for b in range(B):
        L = int(seq_lens[b])
        for h in range(Hkv):
            K, V = gather_unit(k_cache, v_cache, page_table[b], L, h)
            o, lse, _ = verify_unit(q[b, :, h * G:(h + 1) * G], K, V, L, n_q, G, sm_scale)
            O[b, :, h * G:(h + 1) * G] = o.reshape(n_q, G, d)
            LSE[b, :, h * G:(h + 1) * G] = lse.reshape(n_q, G)
    return O, LSE


def block_mass_unit(P, seq_len: int, n_q: int, group: int, block_size: int,
                    score_row_start: int, max_blocks: int):
    """Importance of each KV block of one unit: the probability mass that the
    scored rows put on the block, summed over those rows.  Blocks at or past
    ceil(L / block_size) score 0."""
    scores = np.zeros(max_blocks)
    rows = P[score_row_start * group:n_q * group]
    col_mass = rows.sum(axis=0)                   # [L]
    nblk = (seq_len + block_size - 1) // block_size
    for j in range(nblk):
        scores[j] = col_mass[j * block_size:min((j + 1) * block_size, seq_len)].sum()
    return scores


def verify_with_scores(q, k_cache, v_cache, page_table, seq_lens, sm_scale: float,
                       block_size: int, max_blocks: int, score_row_start: int = 0,
                       units=None):
    """Verify attention plus block scores.

    Returns (O, LSE, block_scores [B][Hkv][max_blocks]).  With ``units`` (a
    list of (b, h) pairs) only those units are computed; the other entries are
    left NaN so that a caller cannot mistake them for results.
    """
    B, n_q, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    O = np.full((B, n_q, Hq, d), np.nan)
    LSE = np.full((B, n_q, Hq), np.nan)
    scores = np.full((B, Hkv, max_blocks), np.nan)
    todo = units if units is not None else [(b, h) for b in range(B) for h in range(Hkv)]
    for b, h in todo:
        L = int(seq_lens[b])
        K, V = gather_unit(k_cache, v_cache, page_table[b], L, h)
        o, lse, P = verify_unit(q[b, :, h * G:(h + 1) * G], K, V, L, n_q, G, sm_scale)
        O[b, :, h * G:(h + 1) * G] = o.reshape(n_q, G, d)
        LSE[b, :, h * G:(h + 1) * G] = lse.reshape(n_q, G)
        scores[b, h] = block_mass_unit(P, L, n_q, G, block_size, score_row_start, max_blocks)
    return O, LSE, scores


# ---------------------------------------------------------------------------
# Top-N block selection (SparseSpec §4.1: Top-K over the aggregated scores)
# ---------------------------------------------------------------------------
def window_start(seq_len: int, window: int) -> int:
    """First token of the recent window; with no window it is L (empty)."""
    if window <= 0:
        return seq_len
    return max(0, seq_len - window)


def topk_unit(scores_row, seq_len: int, block_size: int, budget: int, window: int,
              max_sel: int):
    """Selected block indices (ascending) of one unit.

    Candidates: blocks j < ceil(L/bs) with j * bs < window start.  Order:
    larger score first, lower index first among equal scores.  Keep the first
    min(budget, #candidates, max_sel) of that order.
    """
    ws = window_start(seq_len, window)
    nblk = (seq_len + block_size - 1) // block_size
    cands = [j for j in range(nblk) if j * block_size < ws]
    ranked = sorted(cands, key=lambda j: (-float(scores_row[j]), j))
    keep = ranked[:max(0, min(int(budget), len(cands), max_sel))]
    return sorted(keep)


def block_topk(block_scores, seq_lens, block_size: int, budget, window: int, max_sel: int):
    """Batch Top-N: returns sel [B][Hkv][max_sel] int32 (-1 padded) and
    sel_count [B][Hkv] int32."""
    B, Hkv, _ = block_scores.shape
    sel = np.full((B, Hkv, max_sel), -1, dtype=np.int32)
    cnt = np.zeros((B, Hkv), dtype=np.int32)
    for b in range(B):
        for h in range(Hkv):
            chosen = topk_unit(block_scores[b, h], int(seq_lens[b]), block_size,
                               int(budget[b]), window, max_sel)
            sel[b, h, :len(chosen)] = chosen
            cnt[b, h] = len(chosen)
    return sel, cnt


# ---------------------------------------------------------------------------
# Sparse draft attention (SpecAttn 方法详解: drafting loads only the critical
# entries; SparseSpec §4.1/§4.2: sparse attention over the selected KV)
# ---------------------------------------------------------------------------
def draft_token_set(seq_len: int, sel_row, count: int, block_size: int, window: int):
    """Sorted token positions the draft query attends to."""
    ws = window_start(seq_len, window)
    toks = set()
    for j in sel_row[:count]:
        j = int(j)
        if j < 0:
            continue
        toks.update(range(j * block_size, min((j + 1) * block_size, ws)))
    toks.update(range(ws, seq_len))
    return sorted(toks)


def draft(q, k_cache, v_cache, page_table, seq_lens, sel, sel_count,
          block_size: int, window: int, sm_scale: float, units=None):
    """Single-query sparse attention; q is [B][1][Hq][d].  Returns O
    [B][1][Hq][d] and LSE [B][1][Hq] (fp64)."""
    B, _, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    O = np.full((B, 1, Hq, d), np.nan)
    LSE = np.full((B, 1, Hq), np.nan)
    todo = units if units is not None else [(b, h) for b in range(B) for h in range(Hkv)]
    for b, h in todo:
        L = int(seq_lens[b])
        K, V = gather_unit(k_cache, v_cache, page_table[b], L, h)
        toks = draft_token_set(L, sel[b, h], int(sel_count[b, h]), block_size, window)
        qr = _f64(q[b, 0, h * G:(h + 1) * G])           # [G][d]
        if not toks:
            O[b, 0, h * G:(h + 1) * G] = 0.0
            LSE[b, 0, h * G:(h + 1) * G] = NEG_INF
            continue
        idx = np.asarray(toks)
        S = sm_scale * (qr @ K[idx].T)
        lse, P = _softmax_rows(S)
        O[b, 0, h * G:(h + 1) * G] = P @ V[idx]
        LSE[b, 0, h * G:(h + 1) * G] = lse
    return O, LSE


# ---------------------------------------------------------------------------
# Sparse verification with a layout per query position (SpecSA 核心创新 /
# 重叠感知分组查询执行 and 技术细节与实现挑战 / 稀疏布局的动态管理: every query
# has its own sparse layout; queries whose layouts overlap are run as a group
# that shares the KV blocks.  The grouping changes which loads are shared,
# not what each query computes, so the oracle computes every query alone.)
# ---------------------------------------------------------------------------
def sparse_verify_token_set(seq_len: int, n_q: int, i: int, sel_row, count: int,
                            block_size: int, window: int):
    """Sorted tokens that query position i of a verify step attends to: the
    tokens of its own selected blocks that lie before the window start, plus
    the window, restricted to the causal limit t <= L - n_q + i."""
    count = max(0, min(int(count), len(sel_row)))
    pos = seq_len - n_q + i
    return [t for t in draft_token_set(seq_len, sel_row, count, block_size, window) if t <= pos]


def sparse_verify(q, k_cache, v_cache, page_table, seq_lens, row_sel, row_cnt,
                  block_size: int, window: int, sm_scale: float, units=None):
    """Verify attention in which query position i of request b and KV head h
    attends only to its own layout ``row_sel[b][h][i][:row_cnt[b][h][i]]``
    (block indices; negative entries and blocks at or past the window start
    add nothing) plus the recent window, causally.  Every query head of the
    KV head's group shares the position's layout.

    q: [B][n_q][Hq][d]; row_sel: [B][Hkv][n_q][max_sel]; row_cnt:
    [B][Hkv][n_q].  Returns O [B][n_q][Hq][d] and LSE [B][n_q][Hq] (fp64); an
    empty token set gives O = 0 and LSE = -inf.
    """
    B, n_q, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    O = np.full((B, n_q, Hq, d), np.nan)
    LSE = np.full((B, n_q, Hq), np.nan)
    todo = units if units is not None else [(b, h) for b in range(B) for h in range(Hkv)]
    for b, h in todo:
        L = int(seq_lens[b])
        K, V = gather_unit(k_cache, v_cache, page_table[b], L, h)
        for i in range(n_q):
            toks = sparse_verify_token_set(L, n_q, i, row_sel[b, h, i], int(row_cnt[b, h, i]),
                                           block_size, window)
            heads = slice(h * G, (h + 1) * G)
            if not toks:
                O[b, i, heads] = 0.0
                LSE[b, i, heads] = NEG_INF
                continue
            idx = np.asarray(toks)
            S = sm_scale * (_f64(q[b, i, heads]) @ K[idx].T)   # [G][|toks|]
            lse, P = _softmax_rows(S)
            O[b, i, heads] = P @ V[idx]
            LSE[b, i, heads] = lse
    return O, LSE


def layout_union(row_sel, row_cnt, seq_len: int, block_size: int, window: int):
    """Blocks that at least one query position of a unit selects (before the
    window start), ascending: the blocks a grouped execution loads once."""
    ws = window_start(seq_len, window)
    blocks = set()
    for i in range(row_sel.shape[0]):
        c = max(0, min(int(row_cnt[i]), row_sel.shape[1]))
        for j in row_sel[i, :c]:
            j = int(j)
            if j >= 0 and j * block_size < ws:
                blocks.add(j)
    return sorted(blocks)


# ---------------------------------------------------------------------------
# Split-KV log-sum-exp merge (partials over disjoint KV chunks; SparseSpec
# §4.1 keeps the log-sum-exp of the logits, which is what makes the merge
# possible)
# ---------------------------------------------------------------------------
def merge(o_parts, lse_parts):
    """Combine attention partials over disjoint KV subsets.

    o_parts [S][rows][d], lse_parts [S][rows] -> (O [rows][d], LSE [rows]).
    LSE = log sum_s exp(lse_s); O = sum_s exp(lse_s - LSE) O_s.  Partials with
    LSE -inf carry no weight; if all are -inf the result is O = 0, LSE = -inf.
    """
    o_parts = _f64(o_parts)
    lse_parts = _f64(lse_parts)
    S, rows, d = o_parts.shape
    O = np.zeros((rows, d))
    LSE = np.full(rows, NEG_INF)
    for r in range(rows):
        live = [s for s in range(S) if np.isfinite(lse_parts[s, r])]
        if not live:
            continue
        m = max(lse_parts[s, r] for s in live)
        total = sum(math.exp(lse_parts[s, r] - m) for s in live)
        LSE[r] = m + math.log(total)
        for s in live:
            O[r] += math.exp(lse_parts[s, r] - LSE[r]) * o_parts[s, r]
    return O, LSE


def attention_partial(q_rows, K, V, sm_scale: float, positions, token_ids):
    """(O, LSE) of rows over the token subset ``token_ids`` with causal
    positions ``positions`` (row r sees tokens <= positions[r]).  Used to build
    independent split partials for merge tests."""
    q = _f64(q_rows)
    idx = np.asarray(token_ids, dtype=np.int64)
    S = sm_scale * (q @ K[idx].T) if len(idx) else np.zeros((q.shape[0], 0))
    for r in range(q.shape[0]):
        S[r, idx > positions[r]] = NEG_INF
    lse, P = _softmax_rows(S)
    O = P @ V[idx] if len(idx) else np.zeros((q.shape[0], K.shape[1]))
    return O, lse


# ---------------------------------------------------------------------------
# KV update for the speculative positions (SpecSA 核心创新, 刷新/复用: KV of
# accepted tokens is reused, KV of rejected tokens is refreshed)
# ---------------------------------------------------------------------------
def kv_write(k_cache, v_cache, page_table, k_new, v_new, pos0):
    """Copies of the caches with token ``pos0[b] + i`` of request b set to
    ``k_new[b, i]`` / ``v_new[b, i]`` (all KV heads), through the page table:
    page ``page_table[b][t // page_size]``, slot ``t % page_size``.  A
    position outside the request's table row, or a page id outside the pool,
    leaves the cache unchanged for that token (nothing is written)."""
    k = np.array(k_cache, copy=True)
    v = np.array(v_cache, copy=True)
    num_pages, _, page_size, _ = k.shape
    B, n_new = k_new.shape[0], k_new.shape[1]
    max_pages = page_table.shape[1]
    for b in range(B):
        for i in range(n_new):
            t = int(pos0[b]) + i
            if t < 0 or t // page_size >= max_pages:
                continue
            page = int(page_table[b][t // page_size])
            if page < 0 or page >= num_pages:
                continue
            k[page, :, t % page_size, :] = k_new[b, i]
            v[page, :, t % page_size, :] = v_new[b, i]
    return k, v


def kv_commit(seq_lens, keep, n_q: int):
    """New lengths after verification: the request's last n_q positions were
    the speculative ones; the first ``keep[b]`` of them (clamped to
    [0, n_q]) stay, the rest are dropped.  Their cache slots are not touched:
    a position at or past the length is never read."""
    out = []
    for L, kp in zip(seq_lens, keep):
        kp = min(max(int(kp), 0), n_q)
        out.append(max(int(L) - n_q + kp, 0))
    return np.array(out, dtype=np.int32)
