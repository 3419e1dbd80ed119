"""GPU parity of the fused step (sss_fused_step) against the fp64 oracle,
through the C ABI.

Chained steps (verify -> block scores -> Top-N -> draft of the same
requests) are checked stage by stage: verify outputs and scores against the
oracle; the selection bit-exactly against the oracle's Top-N run on the
step's own fp32 scores; the draft against the oracle's draft over the
step's own selection.  Mixed steps (some requests verify, the others draft
over given selections) are checked the same way.  Small lengths force the
work list to split units into many chunks, so the follow-up launches that
merge, score and select split units run; batches of at least 512 whole
units run the persistent step kernel (its verify, scores and selection are
also checked bitwise against the one-stage-at-a-time calls).
"""
import numpy as np
import pytest
import torch

import harness as H
import oracle
from sparse_self_speculative_sss_amd import workload as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


def mk(name, seed=0, **kw):
    return W.make(name, seed=seed, device=DEV, **kw)


def verify_outputs(wl, vb, with_sel=True):
    B, n_q, hq, _ = vb.q.shape
    hkv = wl.shape.Hkv
    o = torch.full_like(vb.q, float("nan"))
    lse = torch.full((B, n_q, hq), float("nan"), device=DEV)
    sc = torch.full((B, hkv, wl.max_blocks), float("nan"), device=DEV)
    sel = torch.full((B, hkv, wl.max_sel), 777, dtype=torch.int32, device=DEV) if with_sel else None
    cnt = torch.full((B, hkv), -9, dtype=torch.int32, device=DEV) if with_sel else None
    return o, lse, sc, sel, cnt


def run_chained(wl, score_row_start=0, ws=None):
    s = H.sss()
    vb, db = wl.verify, wl.draft
    o, lse, sc, sel, cnt = verify_outputs(wl, vb)
    od = torch.full_like(db.q, float("nan"))
    lsed = torch.full(db.q.shape[:3], float("nan"), device=DEV)
    kv = H.kv_of(wl, vb)
    v = s.verify_step(kv, vb.q, wl.sm_scale, wl.shape.block_size, wl.max_blocks, o, lse, sc,
                      score_row_start=score_row_start, budget=vb.budget, window=wl.shape.window,
                      sel=sel, sel_count=cnt)
    d = s.draft_step(kv, db.q, wl.sm_scale, wl.shape.block_size, sel, cnt, wl.shape.window, od,
                     lsed)
    s.fused_step(v, d, chained=True, ws=ws)
    torch.cuda.synchronize()
    return (o, lse, sc), (sel, cnt), (od, lsed)


def check_selection(wl, batch, sc, sel, cnt, units=None):
    """Selection == oracle Top-N of the step's own fp32 scores (bit-exact)."""
    scores = sc.cpu().numpy().astype(np.float32)
    ref_sel, ref_cnt = oracle.block_topk(scores, batch.seq_lens.cpu().numpy(), wl.shape.block_size,
                                         batch.budget.cpu().numpy(), wl.shape.window, wl.max_sel)
    assert np.array_equal(cnt.cpu().numpy(), ref_cnt)
    assert np.array_equal(sel.cpu().numpy(), ref_sel)
    return sel.cpu().numpy(), cnt.cpu().numpy()


CHAINED = [
    ("qwen_ragged", "qwen3_8b_layer_b16_l4096", dict(B=3, L=300)),
    ("decode_small", "decode_b128_l8192", dict(B=4, L=1000, sigma="one")),
    ("decode_nq1", "qwen3_8b_layer_b16_l4096", dict(B=3, L=77, n_q=1, sigma="one")),
    ("L_eq_nq", "qwen3_8b_layer_b16_l4096", dict(B=2, L=5, window=0, sigma="one")),
    ("d64", "decode_b128_l8192", dict(B=2, L=200, d=64, sigma="one")),
    ("page16_blk64", "qwen3_8b_layer_b16_l4096", dict(B=2, L=700, block_size=64, sigma="one")),
    ("page64_blk64_rows80", "longctx_b4_l128k", dict(B=1, L=2000, sigma="one")),
    ("rows40", "qwen3_8b_layer_b16_l4096", dict(B=2, L=333, Hq=16, Hkv=2, sigma="one")),
    ("rows128", "qwen3_8b_layer_b16_l4096", dict(B=1, L=400, Hq=32, Hkv=1, n_q=4)),
    # 1024 units of whole verify units: verify, Top-N and one-wave draft launches
    ("units1024", "decode_b128_l8192", dict(B=128, L=200, sigma="one")),
]


@pytest.mark.parametrize("case", CHAINED, ids=[c[0] for c in CHAINED])
def test_fused_chained(case):
    cid, name, kw = case
    wl = mk(name, seed=31, **kw)
    vb, db = wl.verify, wl.draft
    hkv = wl.shape.Hkv
    print(f"[fused chained] {cid}", flush=True)
    v_out, (sel, cnt), d_out = run_chained(wl)
    units = H.all_units(vb, hkv)
    H.compare_verify(wl, vb, v_out, units).check(f"fused {cid} verify")
    sc = v_out[2].cpu().numpy()
    for b in range(vb.B):
        nblk = -(-int(vb.seq_lens[b]) // wl.shape.block_size)
        assert np.all(sc[b, :, nblk:] == 0.0)
    sel_np, cnt_np = check_selection(wl, vb, v_out[2], sel, cnt)
    H.compare_draft(wl, db, d_out, sel_np, cnt_np, H.all_units(db, hkv)).check(
        f"fused {cid} draft")


def step_form(wl, chained=True):
    s = H.sss()
    vb, db = wl.verify, wl.draft
    o, lse, sc, sel, cnt = verify_outputs(wl, vb)
    kv = H.kv_of(wl, vb)
    v = s.verify_step(kv, vb.q, wl.sm_scale, wl.shape.block_size, wl.max_blocks, o, lse, sc,
                      budget=vb.budget, window=wl.shape.window, sel=sel, sel_count=cnt)
    d = s.draft_step(kv, db.q, wl.sm_scale, wl.shape.block_size, sel, cnt, wl.shape.window,
                     torch.empty_like(db.q), torch.empty(db.q.shape[:3], device=DEV))
    return s.fused_step_form(v, d, chained)


def nan_equal(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    return bool(((a == b) | (torch.isnan(a) & torch.isnan(b))).all())


@pytest.mark.parametrize("B,L,form", [(128, 512, "two_launch"), (128, 1500, "two_launch"),
                                      (96, 1500, "persistent")])
def test_fused_chained_matches_separate_calls(B, L, form):
    """A chained step of whole units runs the one-launch-per-stage verify's
    arithmetic: verify outputs, scores and selection are bitwise equal.  (A
    batch of 1024 units keeps every unit in one chunk, and its draft runs
    one wave per unit as the separate draft does; smaller batches are split
    to fill the GPU.  At 1500 tokens the block masses make the verify run as
    two-token-group workgroups, two per compute unit; with 768 units the
    step runs persistently: its draft splits each list over two token
    groups, so it equals the separate draft up to summation order.)"""
    wl = mk("decode_b128_l8192", seed=32, B=B, L=L)
    vb = wl.verify
    assert step_form(wl) == form
    v_out, (sel, cnt), d_out = run_chained(wl)
    o, lse, sc = H.gpu_verify(wl, vb, num_splits=1)
    sel2, cnt2 = H.gpu_topk(wl, vb, sc)
    torch.cuda.synchronize()
    assert torch.equal(v_out[0].view(torch.uint8), o.view(torch.uint8))
    assert torch.equal(v_out[1], lse)
    assert torch.equal(v_out[2], sc)
    assert torch.equal(sel, sel2) and torch.equal(cnt, cnt2)
    od, lsed = H.gpu_draft(wl, wl.draft, sel2, cnt2)
    torch.cuda.synchronize()
    if form == "two_launch":
        # 1024 units: the step drafts with the separate draft kernel's arithmetic
        assert torch.equal(d_out[0].view(torch.uint8), od.view(torch.uint8))
        assert torch.equal(d_out[1], lsed)
    else:
        assert torch.isfinite(d_out[0].float()).all() and torch.isfinite(d_out[1]).all()
        assert (d_out[0].float() - od.float()).abs().max().item() <= H.O_MAX_ABS
        assert (d_out[1] - lsed).abs().max().item() <= H.LSE_ABS
        H.compare_draft(wl, wl.draft, d_out, sel.cpu().numpy(), cnt.cpu().numpy(),
                        H.sample_units(wl.draft, wl.shape.Hkv, 24, seed=3)).check(
            "persistent draft")


# Chained steps the persistent kernel runs (512 to 1023 whole units whose
# verify takes two workgroups per compute unit): ragged lengths, a batch
# that is not a multiple of 8 (no XCD-aware order, units not a multiple of
# the grid), blocks of 32 tokens (block masses summed over two segments),
# head dim 64.  Oracle units: "all", or a seeded sample of that many.
PERSIST = [
    ("ragged_b96", "decode_b128_l8192", dict(B=96, L=(1000, 2000), sigma="one"), "all"),
    ("b100_not_mult8", "decode_b128_l8192", dict(B=100, L=1500, sigma="one"), 48),
    ("blk32_b64", "qwen3_8b_layer_b16_l4096", dict(B=64, L=3000, block_size=32, sigma="one"), 32),
    ("d64_b64", "decode_b128_l8192", dict(B=64, L=8400, d=64, sigma="one"), 16),
    ("nq1_b96", "decode_b128_l8192", dict(B=96, L=(5000, 6000), n_q=1, sigma="one"), 32),
]

# Chained steps of 1024 or more whole units of at most 1024 candidates: the
# verify launch, then one wave per unit that selects and drafts over the
# selection it keeps in LDS.  The same shapes as above at 1024+ units, and
# units of exactly 1024 candidates (the largest the one-wave selection takes).
WAVE = [
    ("ragged_b128", "decode_b128_l8192", dict(B=128, L=(1000, 2000), sigma="one"), "all"),
    ("b132_not_mult8", "decode_b128_l8192", dict(B=132, L=1500, sigma="one"), 48),
    ("blk32_b128", "qwen3_8b_layer_b16_l4096", dict(B=128, L=3000, block_size=32, sigma="one"), 32),
    ("d64_b128", "decode_b128_l8192", dict(B=128, L=4100, d=64, sigma="one"), 16),
    ("nq1_b128", "decode_b128_l8192", dict(B=128, L=(5000, 6000), n_q=1, sigma="one"), 32),
    ("cand1024_b128", "decode_b128_l8192", dict(B=128, L=16384, sigma="one"), 8),
]


@pytest.mark.parametrize("case", WAVE, ids=[c[0] for c in WAVE])
def test_fused_select_draft_wave(case):
    cid, name, kw, nunits = case
    wl = mk(name, seed=43, **kw)
    vb, db = wl.verify, wl.draft
    hkv = wl.shape.Hkv
    print(f"[fused select+draft wave] {cid}", flush=True)
    assert step_form(wl) == "two_launch"
    v_out, (sel, cnt), d_out = run_chained(wl)
    # verify, scores, selection and draft: bitwise those of the
    # one-launch-per-stage calls (the separate draft of 1024+ units runs
    # one wave per unit too)
    o, lse, sc = H.gpu_verify(wl, vb, num_splits=1)
    sel2, cnt2 = H.gpu_topk(wl, vb, sc)
    od, lsed = H.gpu_draft(wl, db, sel2, cnt2)
    torch.cuda.synchronize()
    assert torch.equal(v_out[0].view(torch.uint8), o.view(torch.uint8))
    assert torch.equal(v_out[1], lse) and torch.equal(v_out[2], sc)
    assert torch.equal(sel, sel2) and torch.equal(cnt, cnt2)
    assert torch.equal(d_out[0].view(torch.uint8), od.view(torch.uint8))
    assert torch.equal(d_out[1], lsed)
    for t in (*v_out, *d_out):
        assert torch.isfinite(t.float()).all()
    units = H.all_units(vb, hkv) if nunits == "all" else H.sample_units(vb, hkv, nunits, seed=4)
    H.compare_verify(wl, vb, v_out, units).check(f"wave {cid} verify")
    sel_np, cnt_np = check_selection(wl, vb, v_out[2], sel, cnt)
    H.compare_draft(wl, db, d_out, sel_np, cnt_np, units).check(f"wave {cid} draft")


# Chained steps of split units of three row tiles whose verify runs as
# load-wave workgroups: the verify and merge launches, then one workgroup
# per draft chunk that selects its unit's Top-N and drafts the chunk, then
# the draft merge.  80 rows (16-row last tile), ragged lengths (units
# with fewer verify chunks than draft chunks, and units that fit in one
# chunk), 96 rows, 65 rows at head dim 64 with an unsplit draft.
ROWS_SPLIT = [
    ("rows80", "longctx_b4_l128k", dict(B=2, L=3000, sigma="one"), {}),
    ("rows80_ragged", "longctx_b4_l128k", dict(B=3, L=(300, 4000)), {}),
    # requests of 200 and 5 tokens: units in one chunk (finished by their
    # verify workgroup, which then selects)
    ("rows80_short_units", "longctx_b4_l128k", dict(B=4, L=3000, sigma="one"), {1: 200, 3: 5}),
    ("rows96", "longctx_b4_l128k", dict(B=2, L=3000, n_q=6, sigma="one"), {}),
    ("rows65_d64", "qwen3_8b_layer_b16_l4096", dict(B=2, L=3000, Hq=26, Hkv=2, d=64,
                                                    sigma="one"), {}),
    # no recent window (every block a candidate, the list only selected
    # blocks); one block selected; every candidate selected (the selection
    # routine's early return, draft lists of about 190 segments)
    ("rows80_window0", "longctx_b4_l128k", dict(B=2, L=3000, window=0, sigma="one"), {}),
    ("rows80_budget1", "longctx_b4_l128k", dict(B=2, L=3000, budget=1, sigma="one"), {}),
    ("rows80_budget_all", "longctx_b4_l128k", dict(B=2, L=3000, budget=1000, sigma="one"), {}),
]


def separate_calls(wl, kv=None, lens=None):
    """The per-stage calls with their default splits: verify, Top-N, draft."""
    s = H.sss()
    vb, db = wl.verify, wl.draft
    kv = H.kv_of(wl, vb) if kv is None else kv
    lens = vb.seq_lens if lens is None else lens
    bs = wl.shape.block_size
    o, lse, sc, sel, cnt = verify_outputs(wl, vb)
    s.verify_attn(kv, vb.q, wl.sm_scale, bs, wl.max_blocks, o, lse, sc, num_splits=0)
    s.block_topk(sc, lens, bs, vb.budget, wl.shape.window, sel, cnt)
    od = torch.full_like(db.q, float("nan"))
    lsed = torch.full(db.q.shape[:3], float("nan"), device=DEV)
    s.draft_attn(kv, db.q, wl.sm_scale, bs, sel, cnt, wl.shape.window, od, lsed, num_splits=0)
    torch.cuda.synchronize()
    return (o, lse, sc), (sel, cnt), (od, lsed)


@pytest.mark.parametrize("case", ROWS_SPLIT, ids=[c[0] for c in ROWS_SPLIT])
def test_fused_rows_split(case):
    cid, name, kw, short = case
    wl = mk(name, seed=44, **kw)
    vb, db = wl.verify, wl.draft
    for b, n in short.items():
        vb.seq_lens[b] = n
        db.seq_lens[b] = n
    hkv = wl.shape.Hkv
    print(f"[fused rows split] {cid}", flush=True)
    assert step_form(wl) == "rows_split"
    v_out, (sel, cnt), d_out = run_chained(wl)
    # every output bitwise that of the per-stage calls
    v2, (sel2, cnt2), d2 = separate_calls(wl)
    for a, b in zip((*v_out, *d_out), (*v2, *d2)):
        assert nan_equal(a, b)
    assert torch.equal(sel, sel2) and torch.equal(cnt, cnt2)
    for t in (*v_out, *d_out):
        assert torch.isfinite(t.float()).all()
    # a second and third step on the same workspace
    ws = H.sss().workspace(H.sss().fused_workspace_size(*step_args(wl), True), DEV)
    for _ in range(2):
        v3, (sel3, cnt3), d3 = run_chained(wl, ws=ws)
        for a, b in zip((*v3, *d3), (*v2, *d2)):
            assert nan_equal(a, b)
        assert torch.equal(sel3, sel2) and torch.equal(cnt3, cnt2)
    units = H.all_units(vb, hkv)
    H.compare_verify(wl, vb, v_out, units).check(f"rows split {cid} verify")
    sel_np, cnt_np = check_selection(wl, vb, v_out[2], sel, cnt)
    H.compare_draft(wl, db, d_out, sel_np, cnt_np, H.all_units(db, hkv)).check(
        f"rows split {cid} draft")


def step_args(wl):
    s = H.sss()
    vb, db = wl.verify, wl.draft
    o, lse, sc, sel, cnt = verify_outputs(wl, vb)
    kv = H.kv_of(wl, vb)
    v = s.verify_step(kv, vb.q, wl.sm_scale, wl.shape.block_size, wl.max_blocks, o, lse, sc,
                      budget=vb.budget, window=wl.shape.window, sel=sel, sel_count=cnt)
    d = s.draft_step(kv, db.q, wl.sm_scale, wl.shape.block_size, sel, cnt, wl.shape.window,
                     torch.empty_like(db.q), torch.empty(db.q.shape[:3], device=DEV))
    return v, d


def test_fused_rows_split_full_size():
    """The long-context workload at full size (4 requests x 128K tokens, 80
    rows per unit, 64 chunks): every output of the rows-split step bitwise
    that of the per-stage calls (which the full-size parity test checks
    against the oracle on sampled units), all finite."""
    wl = mk("longctx_b4_l128k", seed=47)
    print("[fused rows split] full size", flush=True)
    assert step_form(wl) == "rows_split"
    v_out, (sel, cnt), d_out = run_chained(wl)
    v2, (sel2, cnt2), d2 = separate_calls(wl)
    for a, b in zip((*v_out, *d_out), (*v2, *d2)):
        assert nan_equal(a, b)
        assert torch.isfinite(a.float()).all()
    assert torch.equal(sel, sel2) and torch.equal(cnt, cnt2)


def test_fused_rows_split_poisoned_requests():
    """A request longer than max_seq_len and one with an out-of-range page id
    poison only their own units, bitwise as in the per-stage calls."""
    wl = mk("longctx_b4_l128k", seed=45, B=3, L=3000, sigma="one")
    vb, db = wl.verify, wl.draft
    s = H.sss()
    lens = vb.seq_lens.clone()
    lens[1] = 100000
    table = vb.page_table.clone()
    table[2, 5] = -3
    kv = s.paged_kv(wl.k_cache, wl.v_cache, table, lens, 3000)
    bs = wl.shape.block_size
    o, lse, sc, sel, cnt = verify_outputs(wl, vb)
    od = torch.full_like(db.q, 7.0)
    lsed = torch.full(db.q.shape[:3], 7.0, device=DEV)
    v = s.verify_step(kv, vb.q, wl.sm_scale, bs, wl.max_blocks, o, lse, sc, budget=vb.budget,
                      window=wl.shape.window, sel=sel, sel_count=cnt)
    d = s.draft_step(kv, db.q, wl.sm_scale, bs, sel, cnt, wl.shape.window, od, lsed)
    assert s.fused_step_form(v, d, True) == "rows_split"
    s.fused_step(v, d, chained=True)
    torch.cuda.synchronize()
    v2, (sel2, cnt2), d2 = separate_calls(wl, kv, lens)
    for b in (1, 2):
        for t in (o[b].float(), lse[b], sc[b]):
            assert torch.isnan(t).all()
    assert torch.isnan(od[1].float()).all() and torch.isnan(lsed[1]).all()
    for t in (o[0].float(), lse[0], sc[0], od[0].float(), lsed[0]):
        assert torch.isfinite(t).all()
    for a, b in zip((o, lse, sc, od, lsed), (*v2, *d2)):
        assert nan_equal(a, b)
    assert torch.equal(sel, sel2) and torch.equal(cnt, cnt2)


@pytest.mark.parametrize("case", PERSIST, ids=[c[0] for c in PERSIST])
def test_fused_persistent(case):
    cid, name, kw, nunits = case
    wl = mk(name, seed=41, **kw)
    vb, db = wl.verify, wl.draft
    hkv = wl.shape.Hkv
    print(f"[fused persistent] {cid}", flush=True)
    assert step_form(wl) == "persistent"
    v_out, (sel, cnt), d_out = run_chained(wl)
    # verify arithmetic, scores and selection: bitwise those of the
    # one-launch-per-stage calls
    o, lse, sc = H.gpu_verify(wl, vb, num_splits=1)
    sel2, cnt2 = H.gpu_topk(wl, vb, sc)
    torch.cuda.synchronize()
    assert torch.equal(v_out[0].view(torch.uint8), o.view(torch.uint8))
    assert torch.equal(v_out[1], lse) and torch.equal(v_out[2], sc)
    assert torch.equal(sel, sel2) and torch.equal(cnt, cnt2)
    # every unit's outputs written and finite
    for t in (*v_out, *d_out):
        assert torch.isfinite(t.float()).all()
    units = H.all_units(vb, hkv) if nunits == "all" else H.sample_units(vb, hkv, nunits, seed=4)
    H.compare_verify(wl, vb, v_out, units).check(f"persistent {cid} verify")
    sel_np, cnt_np = check_selection(wl, vb, v_out[2], sel, cnt)
    H.compare_draft(wl, db, d_out, sel_np, cnt_np, units).check(f"persistent {cid} draft")
    # the draft against the separate draft kernel on the same selection, all units
    od, lsed = H.gpu_draft(wl, db, sel2, cnt2)
    torch.cuda.synchronize()
    assert (d_out[0].float() - od.float()).abs().max().item() <= H.O_MAX_ABS
    assert (d_out[1] - lsed).abs().max().item() <= H.LSE_ABS


@pytest.mark.parametrize("B,form", [(64, "persistent"), (128, "two_launch")])
def test_fused_chained_poisoned_requests(B, form):
    """A request longer than max_seq_len and one with an out-of-range page id
    poison only their own units, as in the separate calls (persistent form,
    and the two-launch form with one select-and-draft wave per unit)."""
    wl = mk("decode_b128_l8192", seed=42, B=B, L=1500)
    vb, db = wl.verify, wl.draft
    assert step_form(wl) == form
    s = H.sss()
    lens = vb.seq_lens.clone()
    lens[3] = 100000
    table = vb.page_table.clone()
    table[5, 7] = -3
    kv = s.paged_kv(wl.k_cache, wl.v_cache, table, lens, 1500)
    o, lse, sc, sel, cnt = verify_outputs(wl, vb)
    od = torch.full_like(db.q, 7.0)
    lsed = torch.full(db.q.shape[:3], 7.0, device=DEV)
    v = s.verify_step(kv, vb.q, wl.sm_scale, 16, wl.max_blocks, o, lse, sc, budget=vb.budget,
                      window=wl.shape.window, sel=sel, sel_count=cnt)
    d = s.draft_step(kv, db.q, wl.sm_scale, 16, sel, cnt, wl.shape.window, od, lsed)
    assert s.fused_step_form(v, d, True) == form
    s.fused_step(v, d, chained=True)
    # the same calls one stage at a time
    o2, lse2, sc2 = (torch.empty_like(t) for t in (o, lse, sc))
    s.verify_attn(kv, vb.q, wl.sm_scale, 16, wl.max_blocks, o2, lse2, sc2, num_splits=1)
    sel2, cnt2 = torch.empty_like(sel), torch.empty_like(cnt)
    s.block_topk(sc2, lens, 16, vb.budget, wl.shape.window, sel2, cnt2)
    od2, lsed2 = torch.empty_like(od), torch.empty_like(lsed)
    s.draft_attn(kv, db.q, wl.sm_scale, 16, sel2, cnt2, wl.shape.window, od2, lsed2)
    torch.cuda.synchronize()
    for b in (3, 5):
        for t in (o[b].float(), lse[b], sc[b]):
            assert torch.isnan(t).all()
    assert torch.isnan(od[3].float()).all() and torch.isnan(lsed[3]).all()
    good = [b for b in range(vb.B) if b not in (3, 5)]
    for t in (o[good].float(), lse[good], sc[good], od[good].float(), lsed[good]):
        assert torch.isfinite(t).all()
    assert nan_equal(o, o2) and nan_equal(lse, lse2) and nan_equal(sc, sc2)
    assert torch.equal(sel, sel2) and torch.equal(cnt, cnt2)
    assert torch.equal(torch.isnan(lsed), torch.isnan(lsed2))
    fin = torch.isfinite(lsed)
    assert (lsed[fin] - lsed2[fin]).abs().max().item() <= H.LSE_ABS


# Each fused form repeated on the same inputs and workspace: outputs, scores
# and selections must agree to the bit (the persistent and work-list
# kernels order their waves through LDS, the work list also splits units).
REPEAT = [
    ("two_launch", "decode_b128_l8192", dict(B=128, L=1500, sigma="one")),
    ("persistent", "decode_b128_l8192", dict(B=96, L=(1000, 2000), sigma="one")),
    ("work_list", "qwen3_8b_layer_b16_l4096", dict(B=16, L=(1000, 4096))),
    ("rows_split", "longctx_b4_l128k", dict(B=2, L=3000, sigma="one")),
]


@pytest.mark.parametrize("case", REPEAT, ids=[c[0] for c in REPEAT])
def test_fused_forms_bitwise_repeatable(case):
    form, name, kw = case
    wl = mk(name, seed=46, **kw)
    print(f"[fused repeat] {form}", flush=True)
    assert step_form(wl) == form
    ws = H.sss().workspace(H.sss().fused_workspace_size(*step_args(wl), True), DEV)
    runs = []
    for _ in range(3):
        v_out, (sel, cnt), d_out = run_chained(wl, ws=ws)
        runs.append([t.clone() for t in (*v_out, sel, cnt, *d_out)])
    for r in runs[1:]:
        for a, b in zip(runs[0], r):
            assert nan_equal(a, b)


def test_fused_score_row_start_one():
    wl = mk("qwen3_8b_layer_b16_l4096", seed=33, B=2, L=260, sigma="one")
    vb = wl.verify
    v_out, (sel, cnt), _ = run_chained(wl, score_row_start=1)
    H.compare_verify(wl, vb, v_out, H.all_units(vb, wl.shape.Hkv), score_row_start=1).check(
        "fused r0=1")
    G = wl.shape.Hq // wl.shape.Hkv
    assert np.allclose(v_out[2].cpu().numpy().sum(-1), (wl.shape.n_q - 1) * G, atol=1e-3)


def run_mixed(wl, with_sel=True):
    s = H.sss()
    vb, db = wl.verify, wl.draft
    v = d = None
    v_out = d_out = None
    if vb is not None:
        o, lse, sc, sel, cnt = verify_outputs(wl, vb, with_sel)
        v = s.verify_step(H.kv_of(wl, vb), vb.q, wl.sm_scale, wl.shape.block_size, wl.max_blocks,
                          o, lse, sc, budget=vb.budget if with_sel else None,
                          window=wl.shape.window, sel=sel, sel_count=cnt)
        v_out = (o, lse, sc, sel, cnt)
    if db is not None:
        od = torch.full_like(db.q, float("nan"))
        lsed = torch.full(db.q.shape[:3], float("nan"), device=DEV)
        d = s.draft_step(H.kv_of(wl, db), db.q, wl.sm_scale, wl.shape.block_size, db.sel,
                         db.sel_count, wl.shape.window, od, lsed)
        d_out = (od, lsed)
    s.fused_step(v, d, chained=False)
    torch.cuda.synchronize()
    return v_out, d_out


MIXED = [
    ("mixed_small", dict(B=12, L=(200, 3000), sigma="one"), True),
    ("mixed_scores_only", dict(B=10, L=(50, 1500)), False),
    ("mixed_long", dict(B=6, L=(3000, 9000)), True),
]


@pytest.mark.parametrize("case", MIXED, ids=[c[0] for c in MIXED])
def test_fused_mixed(case):
    cid, kw, with_sel = case
    wl = mk("mixed_b96_l1k_32k", seed=34, p_verify=0.4, **kw)
    vb, db = wl.verify, wl.draft
    hkv = wl.shape.Hkv
    print(f"[fused mixed] {cid} verify={vb.B if vb else 0} draft={db.B if db else 0}", flush=True)
    v_out, d_out = run_mixed(wl, with_sel)
    if vb is not None:
        H.compare_verify(wl, vb, v_out[:3], H.all_units(vb, hkv)).check(f"fused {cid} verify")
        if with_sel:
            check_selection(wl, vb, v_out[2], v_out[3], v_out[4])
    if db is not None:
        H.compare_draft(wl, db, d_out, db.sel.cpu().numpy(), db.sel_count.cpu().numpy(),
                        H.all_units(db, hkv)).check(f"fused {cid} draft")


def test_fused_draft_only_split_lists():
    """Draft-only step with long lists: each unit's list is cut into several
    chunks, which the follow-up merge launch combines."""
    wl = mk("qwen3_8b_layer_b16_l4096", seed=35, B=3, L=2900, sigma="one")
    db = wl.draft
    hkv = wl.shape.Hkv
    bs, win = wl.shape.block_size, wl.shape.window
    lens = db.seq_lens.cpu().numpy()
    max_sel = wl.max_blocks
    sel = np.full((db.B, hkv, max_sel), -1, np.int32)
    cnt = np.zeros((db.B, hkv), np.int32)
    g = np.random.default_rng(5)
    for b in range(db.B):
        ncand = -(-max(0, int(lens[b]) - win) // bs)
        for h in range(hkv):
            n = int(g.integers(ncand // 2, ncand + 1))
            pick = np.sort(g.choice(ncand, n, replace=False))
            sel[b, h, :n] = pick
            cnt[b, h] = n
    sel_t, cnt_t = torch.from_numpy(sel).to(DEV), torch.from_numpy(cnt).to(DEV)
    od = torch.full_like(db.q, float("nan"))
    lsed = torch.full(db.q.shape[:3], float("nan"), device=DEV)
    s = H.sss()
    d = s.draft_step(H.kv_of(wl, db), db.q, wl.sm_scale, bs, sel_t, cnt_t, win, od, lsed)
    s.fused_step(None, d, chained=False)
    torch.cuda.synchronize()
    H.compare_draft(wl, db, (od, lsed), sel, cnt, H.all_units(db, hkv)).check("fused draft split")


def test_fused_determinism():
    wl = mk("mixed_b96_l1k_32k", seed=36, p_verify=0.5, B=10, L=(100, 4000))
    runs = []
    for _ in range(2):
        v_out, d_out = run_mixed(wl)
        runs.append([t.cpu() for t in (*v_out, *d_out)])
    wl2 = mk("qwen3_8b_layer_b16_l4096", seed=37, B=3, L=1500)
    for _ in range(2):
        v_out, sel_out, d_out = run_chained(wl2)
        runs.append([t.cpu() for t in (*v_out, *sel_out, *d_out)])
    for i, j in ((0, 1), (2, 3)):
        for a, b in zip(runs[i], runs[j]):
            if a.dtype == torch.bfloat16:
                a, b = a.view(torch.uint8), b.view(torch.uint8)
            assert torch.equal(a, b)


def test_fused_invalid_seq_len_poisons_outputs():
    wl = mk("qwen3_8b_layer_b16_l4096", seed=38, B=3, L=200)
    vb, db = wl.verify, wl.draft
    lens = vb.seq_lens.clone()
    lens[1] = 100000                 # above max_seq_len
    s = H.sss()
    kv = s.paged_kv(wl.k_cache, wl.v_cache, vb.page_table, lens, 200)
    o, lse, sc, sel, cnt = verify_outputs(wl, vb)
    od = torch.zeros_like(db.q)
    lsed = torch.zeros(db.q.shape[:3], device=DEV)
    v = s.verify_step(kv, vb.q, wl.sm_scale, 16, wl.max_blocks, o, lse, sc, budget=vb.budget,
                      window=wl.shape.window, sel=sel, sel_count=cnt)
    d = s.draft_step(kv, db.q, wl.sm_scale, 16, sel, cnt, wl.shape.window, od, lsed)
    s.fused_step(v, d, chained=True)
    torch.cuda.synchronize()
    for t in (o[1].float(), lse[1], sc[1], od[1].float(), lsed[1]):
        assert torch.isnan(t).all()
    for t in (o[0].float(), lse[0], sc[0], od[2].float(), lsed[2]):
        assert torch.isfinite(t).all()


def test_fused_full_size_sampled():
    """The benchmark workloads the fused step serves, in the benchmark's
    launch configuration, on a seeded sample of units (selection bit-exact
    against the oracle's Top-N of the step's own scores for chained steps)."""
    for name in ("decode_b128_l8192", "mixed_b96_l1k_32k", "qwen3_8b_layer_b16_l4096"):
        wl = mk(name, seed=0)
        hkv = wl.shape.Hkv
        vb, db = wl.verify, wl.draft
        print(f"[fused full] {name}", flush=True)
        if wl.shape.p_verify is None:
            v_out, (sel, cnt), d_out = run_chained(wl)
            sel_np, cnt_np = check_selection(wl, vb, v_out[2], sel, cnt)
            vo = v_out
        else:
            v_out, d_out = run_mixed(wl)
            vo = v_out[:3]
            sel_np, cnt_np = db.sel.cpu().numpy(), db.sel_count.cpu().numpy()
        units = H.sample_units(vb, hkv, 6, seed=1)
        H.compare_verify(wl, vb, vo, units).check(f"fused {name} verify")
        G = wl.shape.Hq // hkv
        tot = vo[2].sum(-1).cpu().numpy()
        assert np.abs(tot - wl.shape.n_q * G).max() < 5e-3
        d_units = H.sample_units(db, hkv, 6, seed=2)
        H.compare_draft(wl, db, d_out, sel_np, cnt_np, d_units).check(f"fused {name} draft")


@pytest.mark.parametrize("name,kw,form", [
    ("decode_b128_l8192", dict(B=128, L=1500), "two_launch"),
    ("decode_b128_l8192", dict(B=64, L=1500), "persistent"),
    ("qwen3_8b_layer_b16_l4096", dict(B=16, L=2000), "work_list"),
])
def test_fused_step_marked(name, kw, form):
    """sss_fused_step_marked records the caller's event between the step's
    start and end (after the launch producing the verify outputs) and
    computes exactly what sss_fused_step computes."""
    wl = mk(name, seed=44, **kw)
    assert step_form(wl) == form
    ref_v, ref_sel, ref_d = run_chained(wl)
    s = H.sss()
    vb, db = wl.verify, wl.draft
    o, lse, sc, sel, cnt = verify_outputs(wl, vb)
    od = torch.full_like(db.q, float("nan"))
    lsed = torch.full(db.q.shape[:3], float("nan"), device=DEV)
    kv = H.kv_of(wl, vb)
    v = s.verify_step(kv, vb.q, wl.sm_scale, wl.shape.block_size, wl.max_blocks, o, lse, sc,
                      budget=vb.budget, window=wl.shape.window, sel=sel, sel_count=cnt)
    d = s.draft_step(kv, db.q, wl.sm_scale, wl.shape.block_size, sel, cnt, wl.shape.window, od,
                     lsed)
    start, mid, end = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    mid.record()  # creates the event the library records again
    torch.cuda.synchronize()
    start.record()
    s.fused_step(v, d, chained=True, verify_done=mid._as_parameter_)
    end.record()
    torch.cuda.synchronize()
    assert start.elapsed_time(mid) > 0 and mid.elapsed_time(end) >= 0
    for a, b in zip((o, lse, sc, sel, cnt, od, lsed), (*ref_v, *ref_sel, *ref_d)):
        assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.uint8) if b.dtype == torch.bfloat16 else b)
