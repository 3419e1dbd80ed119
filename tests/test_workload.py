"""Seeded input generator: determinism and structure (no attention maths)."""
import math

import torch

from sparse_self_speculative_sss_amd import workload as W


def test_same_seed_same_inputs():
    a = W.make("qwen3_8b_layer_b16_l4096", seed=3, B=2, L=300)
    b = W.make("qwen3_8b_layer_b16_l4096", seed=3, B=2, L=300)
    c = W.make("qwen3_8b_layer_b16_l4096", seed=4, B=2, L=300)
    assert torch.equal(a.k_cache, b.k_cache) and torch.equal(a.v_cache, b.v_cache)
    assert torch.equal(a.verify.q, b.verify.q) and torch.equal(a.verify.page_table, b.verify.page_table)
    assert not torch.equal(a.k_cache, c.k_cache)


def test_page_table_is_a_permutation_and_budgets():
    wl = W.make("mixed_b96_l1k_32k", seed=1, B=20, L=(40, 500))
    lens = wl.seq_lens_all
    P = wl.shape.page_size
    pages = []
    for bt in (wl.verify, wl.draft):
        if bt is None:
            continue
        for i, b in enumerate(bt.req_ids):
            n = -(-lens[b] // P)
            pages += bt.page_table[i, :n].tolist()
            assert int(bt.budget[i]) == math.ceil(0.05 * (-(-lens[b] // 16)))
    assert sorted(pages) == list(range(wl.k_cache.shape[0]))
    assert all(40 <= x <= 500 for x in lens)
    # given draft lists are distinct, ascending candidates
    d = wl.draft
    for i, b in enumerate(d.req_ids):
        ws = max(0, lens[b] - 64)
        for h in range(wl.shape.Hkv):
            s = d.sel[i, h, :int(d.sel_count[i, h])].tolist()
            assert s == sorted(set(s)) and all(j * 16 < ws for j in s)


def test_draft_query_is_last_verify_row():
    wl = W.make("decode_b128_l8192", seed=0, B=2, L=200)
    assert torch.equal(wl.draft.q[:, 0], wl.verify.q[:, -1])


def test_clustered_blocks_planting():
    wl = W.make("longctx_b4_l128k", seed=2, B=1, L=64 * 400)
    pos = wl.extras["planted"][(0, 0)]
    blocks = sorted({p // 64 for p in pos})
    assert len(pos) == 64 * len(blocks) and len(blocks) == 2 * max(1, round(0.005 * 400) // 2)
