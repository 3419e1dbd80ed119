"""GPU parity of sparse verification (a layout per query position,
sss_sparse_verify_attn) against the oracle, through the C ABI: every unit of
reduced shapes across the kernel's row-tile configurations, split merges,
windows shorter than the step, empty sets, malformed layout entries, and a
sample of the full-size workload in the benchmark's launch configuration."""
import numpy as np
import pytest
import torch

import harness as H
from sparse_self_speculative_sss_amd import workload as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


def mk(name, seed=0, **kw):
    return W.make(name, seed=seed, device=DEV, **kw)


# (id, shape, overrides, num_splits list, windows)
CASES = [
    ("rows20", "sparsever_b128_l8192", dict(B=3, L=700, sigma="one"), [0, 1, 3], [64, 0]),
    ("rows20_shared0", "sparsever_b128_l8192", dict(B=2, L=900, layout_shared=0.0), [0, 2], [64]),
    ("rows20_shared1", "sparsever_b128_l8192", dict(B=2, L=900, layout_shared=1.0), [0], [64]),
    ("rows20_w2", "sparsever_b128_l8192", dict(B=2, L=333, sigma="one"), [0, 2], [2]),
    ("nq1", "sparsever_b128_l8192", dict(B=2, L=400, n_q=1, sigma="one"), [0, 2], [64, 0]),
    ("rows40", "sparsever_b128_l8192", dict(B=2, L=500, Hq=16, Hkv=2, sigma="one"), [0, 2], [64]),
    ("rows80_blk64", "longctx_b4_l128k", dict(B=1, L=3000, sigma="one", layout_shared=0.5),
     [0, 4], [128, 3]),
    ("rows128", "sparsever_b128_l8192", dict(B=1, L=600, Hq=32, Hkv=1, n_q=4), [0, 2], [64]),
    ("d64", "sparsever_b128_l8192", dict(B=2, L=300, d=64, sigma="one"), [0, 1], [64]),
    ("page32", "sparsever_b128_l8192", dict(B=2, L=450, page_size=32, sigma="one"), [0], [64]),
    ("L_eq_nq", "sparsever_b128_l8192", dict(B=2, L=5, window=0, sigma="one"), [0], [0, 3]),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_sparse_verify_small(case):
    cid, name, kw, splits, windows = case
    if "layout_shared" not in kw:
        kw = dict(kw, layout_shared=0.7)
    wl = mk(name, seed=31, **kw)
    vb = wl.verify
    rs, rc = vb.row_sel, vb.row_sel_count
    rs_np, rc_np = rs.cpu().numpy(), rc.cpu().numpy()
    units = H.all_units(vb, wl.shape.Hkv)
    for ns in splits:
        for window in windows:
            print(f"[sparse] {cid} num_splits={ns} window={window}", flush=True)
            out = H.gpu_sparse_verify(wl, vb, rs, rc, num_splits=ns, window=window)
            torch.cuda.synchronize()
            H.compare_sparse(wl, vb, out, rs_np, rc_np, units, window=window).check(
                f"sparse {cid} splits={ns} W={window}")


def test_sparse_verify_malformed_entries_and_counts():
    """Negative entries, blocks at or past the window start, repeats, counts
    beyond max_sel and negative counts are read as the definition says."""
    wl = mk("sparsever_b128_l8192", seed=32, B=2, L=2000, sigma="one", layout_shared=0.5)
    vb = wl.verify
    rs = vb.row_sel.clone()
    rc = vb.row_sel_count.clone()
    nblk = -(-2000 // 16)
    rs[0, 0, 0, 0] = -5
    rs[0, 1, 2, 1] = nblk - 1            # inside the window: adds nothing
    rs[0, 1, 2, 2] = nblk + 100          # past the sequence
    rs[1, 0, 3, :] = rs[1, 0, 3, 0]      # one block repeated
    rc[1, 2, 1] = 10 ** 6                # clamped to max_sel
    rc[1, 3, 4] = -4                     # no blocks
    rc[0, 2, :] = 0                      # a unit with the window only
    for ns in (0, 3):
        print(f"[sparse] malformed num_splits={ns}", flush=True)
        out = H.gpu_sparse_verify(wl, vb, rs, rc, num_splits=ns)
        torch.cuda.synchronize()
        H.compare_sparse(wl, vb, out, rs.cpu().numpy(), np.clip(rc.cpu().numpy(), None, 10 ** 6),
                         H.all_units(vb, wl.shape.Hkv)).check(f"malformed splits={ns}")


def test_sparse_verify_empty_sets():
    """No window and nothing selected: every row is O = 0, LSE = -inf."""
    wl = mk("sparsever_b128_l8192", seed=33, B=2, L=200)
    vb = wl.verify
    rc = torch.zeros_like(vb.row_sel_count)
    for ns in (0, 2):
        o, lse = H.gpu_sparse_verify(wl, vb, vb.row_sel, rc, num_splits=ns, window=0)
        torch.cuda.synchronize()
        assert torch.all(o.float() == 0) and torch.all(torch.isneginf(lse))


def test_sparse_verify_full_layouts_match_dense_verify():
    """Every candidate block in every layout: the result is the dense verify
    kernel's (same inputs, both within tolerance of the oracle, and close to
    each other)."""
    wl = mk("sparsever_b128_l8192", seed=34, B=2, L=517, sigma="one")
    vb = wl.verify
    nblk = -(-517 // 16)
    B, hkv, n_q = vb.row_sel_count.shape
    rs = torch.arange(nblk, dtype=torch.int32, device=DEV).expand(B, hkv, n_q, nblk).contiguous()
    rc = torch.full((B, hkv, n_q), nblk, dtype=torch.int32, device=DEV)
    o_s, lse_s = H.gpu_sparse_verify(wl, vb, rs, rc, num_splits=2)
    o_d, lse_d, _ = H.gpu_verify(wl, vb, num_splits=2)
    torch.cuda.synchronize()
    assert (o_s.float() - o_d.float()).abs().max().item() < 2e-2
    assert (lse_s - lse_d).abs().max().item() < 1e-3


def test_sparse_verify_invalid_length_poisons_outputs():
    wl = mk("sparsever_b128_l8192", seed=35, B=2, L=100)
    vb = wl.verify
    bad = vb.seq_lens.clone()
    bad[1] = wl.shape.n_q - 1            # shorter than the step
    kv = H.sss().paged_kv(wl.k_cache, wl.v_cache, vb.page_table, bad, vb.max_seq_len)
    B, n_q, hq, d = vb.q.shape
    for ns in (0, 2):
        o = torch.zeros_like(vb.q)
        lse = torch.zeros((B, n_q, hq), device=DEV)
        H.sss().sparse_verify_attn(kv, vb.q, wl.sm_scale, 16, vb.row_sel, vb.row_sel_count,
                                   wl.shape.window, o, lse, num_splits=ns)
        torch.cuda.synchronize()
        assert torch.all(torch.isnan(o[1].float())) and torch.all(torch.isnan(lse[1]))
        assert torch.all(torch.isfinite(o[0].float())) and torch.all(torch.isfinite(lse[0]))


def test_sparse_verify_full_size_sampled():
    wl = mk("sparsever_b128_l8192", seed=0)
    vb = wl.verify
    print("[sparse] full size", flush=True)
    out = H.gpu_sparse_verify(wl, vb, vb.row_sel, vb.row_sel_count, num_splits=wl.shape.num_splits)
    torch.cuda.synchronize()
    units = H.sample_units(vb, wl.shape.Hkv, 8, seed=3)
    H.compare_sparse(wl, vb, out, vb.row_sel.cpu().numpy(), vb.row_sel_count.cpu().numpy(),
                     units).check("sparse full size")
    # outputs of every unit are finite
    assert torch.all(torch.isfinite(out[0].float())) and torch.all(torch.isfinite(out[1]))
