"""sss_verify_attn_noalloc (static device scratch, no workspace argument)
against sss_verify_attn with a caller workspace, through the C ABI.

Both run the same plan and kernels, so the outputs must be bitwise equal.
The calls come in a row on one GPU, each smaller than the one before, so
the second and third read a scratch that still holds the previous call's
partials and block masses.
"""
import ctypes

import pytest
import torch

from sparse_self_speculative_sss_amd import sss
from sparse_self_speculative_sss_amd import workload as W

pytestmark = pytest.mark.gpu
DEV = "cuda"

# (shape, overrides, num_splits): split units (partials and block masses in
# the scratch), then a smaller split call, then single-token blocks (every
# token's logits in the scratch, one chunk per unit)
CALLS = [
    ("decode_b128_l8192", dict(B=4, L=3000), 4),
    ("qwen3_8b_layer_b16_l4096", dict(B=2, L=700, sigma="one"), 2),
    ("tokensel_b128_l8192", dict(B=2, L=517, sigma="one"), 0),
]


def _outputs(wl):
    vb, s = wl.verify, wl.shape
    o = torch.full_like(vb.q, float("nan"))
    lse = torch.full((vb.B, s.n_q, s.Hq), float("nan"), dtype=torch.float32, device=DEV)
    sc = torch.full((vb.B, s.Hkv, wl.max_blocks), float("nan"), dtype=torch.float32, device=DEV)
    return o, lse, sc


def _run_pair(name, kw, splits):
    wl = W.make(name, seed=3, device=DEV, **kw)
    vb, s = wl.verify, wl.shape
    kv = sss.paged_kv(wl.k_cache, wl.v_cache, vb.page_table, vb.seq_lens, vb.max_seq_len)
    need = sss.verify_workspace_size(kv, vb.B, s.n_q, s.Hq, s.block_size, wl.max_blocks, splits)
    assert 0 < need <= sss.NOALLOC_SCRATCH_BYTES, (name, need)
    ref = _outputs(wl)
    sss.verify_attn(kv, vb.q, wl.sm_scale, s.block_size, wl.max_blocks, *ref,
                    num_splits=splits)
    got = _outputs(wl)
    sss.verify_attn_noalloc(kv, vb.q, wl.sm_scale, s.block_size, wl.max_blocks, *got,
                            num_splits=splits)
    torch.cuda.synchronize()
    for what, a, b in zip(("o", "lse", "block_scores"), got, ref):
        assert torch.isfinite(b).all(), (name, what)
        assert torch.equal(a, b), (name, what, (a.float() - b.float()).abs().max().item())


def test_noalloc_equals_workspace_call_in_a_row():
    for name, kw, splits in CALLS:
        print(f"noalloc: {name} {kw} splits={splits}", flush=True)
        _run_pair(name, kw, splits)


def test_noalloc_rejects_a_call_beyond_its_scratch():
    # 8 requests x 128K tokens x 2 KV heads x 80 rows in 64 chunks need
    # ~26 MB of partials and ~5 MB of block masses per 4 requests: 8
    # requests exceed the 32 MiB
    kv = sss.PagedKV(k=256, v=512, dtype=sss.SSS_BF16, num_pages=16384, page_size=64,
                     num_kv_heads=2, head_dim=128, max_pages_per_req=2048, page_table=1024,
                     seq_lens=2048, max_seq_len=131072)
    need = sss.verify_workspace_size(kv, 8, 5, 32, 64, 2048, 64)
    assert need > sss.NOALLOC_SCRATCH_BYTES
    lib = sss.raw()
    st = lib.sss_verify_attn_noalloc(ctypes.byref(kv), 4096, 8, 5, 32, 0.088, 64, 0, 64, 8192,
                                     16384, 32768, 2048, None)
    assert st == sss.SSS_ERR_WORKSPACE_TOO_SMALL
    assert b"sss_verify_attn_noalloc" in lib.sss_last_error()
