"""Negative controls for the parity checks (CPU, no GPU).

The parity tests compare the HIP path with the oracle through
harness.compare_* and Stats.check.  Here the oracle's own outputs stand in
for the HIP path: they must pass the checks, and planted defects must fail
them.  Whether the absolute bound on O rejects an all-zero O depends on the
scale of O (near-uniform attention over values ~ N(0, 1/d) gives outputs of
order 1e-3); the relative-L2 diagnostic rejects it at any scale.
"""
import numpy as np
import pytest
import torch

import harness as H
from sparse_self_speculative_sss_amd import workload as W


def _oracle_as_gpu(wl, batch, units):
    """Oracle verify outputs laid out like the HIP path's (O rounded to bf16)."""
    B, n_q, hq, d = batch.q.shape
    hkv = wl.shape.Hkv
    o = torch.zeros((B, n_q, hq, d), dtype=torch.float64)
    lse = torch.zeros((B, n_q, hq), dtype=torch.float64)
    sc = torch.zeros((B, hkv, wl.max_blocks), dtype=torch.float64)
    for (b, h), (Or, LSEr, Sr) in H.oracle_verify_units(wl, batch, units).items():
        gs = H.group_slice(wl, h)
        o[b, :, gs] = torch.from_numpy(Or[:, gs])
        lse[b, :, gs] = torch.from_numpy(LSEr[:, gs])
        sc[b, h] = torch.from_numpy(Sr)
    return o.to(torch.bfloat16), lse.float(), sc.float()


@pytest.fixture(scope="module")
def case():
    wl = W.make("decode_b128_l8192", seed=5, device="cpu", B=2, L=300)
    vb = wl.verify
    units = H.all_units(vb, wl.shape.Hkv)
    return wl, vb, units, _oracle_as_gpu(wl, vb, units)


def _fails(wl, vb, units, out):
    with pytest.raises(AssertionError):
        H.compare_verify(wl, vb, out, units).check("planted defect")


def test_oracle_outputs_pass(case):
    wl, vb, units, out = case
    H.compare_verify(wl, vb, out, units).check("oracle as the HIP path")


def test_all_zero_o_fails(case):
    wl, vb, units, (o, lse, sc) = case
    zero = torch.zeros_like(o)
    st = H.compare_verify(wl, vb, (zero, lse, sc), units)
    # relative L2 error of an all-zero O is 1 whatever the scale of O
    assert abs(st.rel_l2 - 1.0) < 1e-12 and st.rel_l2 > H.O_REL_L2
    _fails(wl, vb, units, (zero, lse, sc))


def test_shifted_o_fails(case):
    wl, vb, units, (o, lse, sc) = case
    bad = o.float().clone()
    bad[1, 2, 5, 17] += 0.05
    _fails(wl, vb, units, (bad.to(torch.bfloat16), lse, sc))


def test_lse_off_fails(case):
    wl, vb, units, (o, lse, sc) = case
    bad = lse.clone()
    bad[0, 4, 30] += 2e-3
    _fails(wl, vb, units, (o, bad, sc))


def test_block_score_off_fails(case):
    wl, vb, units, (o, lse, sc) = case
    bad = sc.clone()
    bad[1, 3, 7] += 2e-3
    _fails(wl, vb, units, (o, lse, bad))


def test_swapped_heads_fail(case):
    """O of two query heads of one group exchanged (a wrong GQA row map)."""
    wl, vb, units, (o, lse, sc) = case
    bad = o.clone()
    bad[:, :, [0, 1]] = o[:, :, [1, 0]]
    _fails(wl, vb, units, (bad, lse, sc))


def test_all_zero_draft_fails():
    wl = W.make("decode_b128_l8192", seed=6, device="cpu", B=2, L=300)
    vb, db = wl.verify, wl.draft
    units = H.all_units(db, wl.shape.Hkv)
    _, sel, cnt = H.oracle_selection(wl, vb, units)
    ref = H.oracle_draft_units(wl, db, sel, cnt, units)
    B, _, hq, d = db.q.shape
    o = torch.zeros((B, 1, hq, d), dtype=torch.float64)
    lse = torch.zeros((B, 1, hq), dtype=torch.float64)
    for (b, h), (Or, LSEr) in ref.items():
        gs = H.group_slice(wl, h)
        o[b, :, gs] = torch.from_numpy(Or[:, gs])
        lse[b, :, gs] = torch.from_numpy(LSEr[:, gs])
    H.compare_draft(wl, db, (o.to(torch.bfloat16), lse.float()), sel, cnt, units).check("oracle draft")
    with pytest.raises(AssertionError):
        H.compare_draft(wl, db, (torch.zeros_like(o).to(torch.bfloat16), lse.float()), sel, cnt,
                        units).check("all-zero draft O")
