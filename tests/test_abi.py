"""The C-ABI library loads without a GPU, exports every declared entry point,
and rejects invalid arguments on the host before launching anything."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "sparse_self_speculative_sss_amd", "libsss.so")
HDR = os.path.join(ROOT, "include", "sss.h")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libsss.so not built")


def declared():
    """Every sss_* function any header in include/ declares."""
    inc = os.path.join(ROOT, "include")
    text = "".join(open(os.path.join(inc, f)).read() for f in sorted(os.listdir(inc))
                   if f.endswith(".h"))
    return sorted(set(re.findall(r"\b(sss_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    names = declared()
    assert {"sss_verify_attn", "sss_block_topk", "sss_draft_attn", "sss_merge",
            "sss_verify_attn_noalloc", "sss_probe_stream_read", "sss_probe_paged_read"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    out = os.popen(f"nm -D --defined-only {LIB}").read()
    for n in names:
        assert re.search(rf"\bT {n}\b", out), n


def _binding():
    from sparse_self_speculative_sss_amd import sss
    return sss


def good_kv(sss, **kw):
    base = dict(k=256, v=512, dtype=sss.SSS_BF16, num_pages=64, page_size=16, num_kv_heads=2,
                head_dim=128, max_pages_per_req=8, page_table=1024, seq_lens=2048,
                max_seq_len=128)
    base.update(kw)
    return sss.PagedKV(**base)


def call_verify(sss, kv, **kw):
    a = dict(q=4096, batch=2, n_q=5, hq=8, scale=0.1, bs=16, r0=0, splits=0, o=8192, lse=16384,
             sc=32768, mb=8, ws=65536, wsb=1 << 30)
    a.update(kw)
    return sss.raw().sss_verify_attn(ctypes.byref(kv), a["q"], a["batch"], a["n_q"], a["hq"],
                                     a["scale"], a["bs"], a["r0"], a["splits"], a["o"], a["lse"],
                                     a["sc"], a["mb"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kvkw,callkw,status", [
    (dict(head_dim=96), {}, 2),
    (dict(dtype=7), {}, 2),
    (dict(page_size=0), {}, 1),
    (dict(max_pages_per_req=4), {}, 1),          # 4 * 16 < 128
    (dict(k=258), {}, 1),                        # misaligned cache
    ({}, dict(n_q=0), 1),
    ({}, dict(n_q=33), 1),
    ({}, dict(hq=7), 1),                         # not a multiple of Hkv
    ({}, dict(hq=128, n_q=5), 2),                # 5 * 64 rows > 128
    ({}, dict(bs=0), 1),
    ({}, dict(mb=7), 1),                         # < ceil(128 / 16)
    ({}, dict(r0=5), 1),
    ({}, dict(splits=-1), 1),
    ({}, dict(scale=float("inf")), 1),
    ({}, dict(q=4100), 1),                       # misaligned q
    ({}, dict(o=0), 1),
    (dict(max_seq_len=1024, max_pages_per_req=64), dict(mb=64, wsb=16, splits=4), 3),
    # (split units need a workspace for their partials: too small, misaligned)
    (dict(max_seq_len=1024, max_pages_per_req=64), dict(mb=64, ws=65537, splits=4), 1),
])
def test_verify_rejects_bad_arguments(kvkw, callkw, status):
    sss = _binding()
    kv = good_kv(sss, **kvkw)
    assert call_verify(sss, kv, **callkw) == status
    assert sss.raw().sss_last_error()


def test_workspace_queries():
    sss = _binding()
    kv = good_kv(sss)
    n = sss.verify_workspace_size(kv, 2, 5, 8, 16, 8, 0)
    assert n >= 0 and n % 256 == 0
    long_kv = good_kv(sss, max_seq_len=1024, max_pages_per_req=64)
    n4 = sss.verify_workspace_size(long_kv, 2, 5, 8, 16, 64, 4)
    assert n4 > 0 and n4 % 256 == 0
    assert sss.draft_workspace_size(kv, 2, 8, 16, 4, 64, 1) >= 0
    with pytest.raises(sss.SSSError):
        sss.verify_workspace_size(good_kv(sss, head_dim=65), 2, 5, 8, 16, 8, 0)


def test_other_entry_points_reject_bad_arguments():
    sss = _binding()
    lib = sss.raw()
    assert lib.sss_block_topk(256, 1, 0, 8, 256, 16, 256, 0, 256, 256, 4, None) == 1
    assert lib.sss_block_topk(256, 1, 2, 8, 256, 16, 256, -1, 256, 256, 4, None) == 1
    assert lib.sss_block_topk(256, 1, 2, 8, 256, 16, 256, 0, 256, 256, 0, None) == 1
    assert lib.sss_block_topk(None, 1, 2, 8, 256, 16, 256, 0, 256, 256, 4, None) == 1
    kv = good_kv(sss)
    d = lib.sss_draft_attn
    assert d(ctypes.byref(kv), 4096, 2, 8, 0.1, 16, 256, 256, 0, 64, 0, 8192, 256, 65536, 1 << 20, None) == 1
    assert d(ctypes.byref(kv), 4096, 2, 8, 0.1, 16, 256, 256, 4, -1, 0, 8192, 256, 65536, 1 << 20, None) == 1
    assert d(ctypes.byref(kv), 4096, 2, 7, 0.1, 16, 256, 256, 4, 64, 0, 8192, 256, 65536, 1 << 20, None) == 1
    m = lib.sss_merge
    assert m(256, 256, 0, 4, 128, 256, 0, 256, None) == 1
    assert m(256, 256, 2, 4, 0, 256, 0, 256, None) == 1
    assert m(256, 256, 2, 4, 128, 256, 9, 256, None) == 2
    # zero-size work is a successful no-op (nothing to launch)
    assert m(256, 256, 2, 0, 128, 256, 0, 256, None) == 0
    assert call_verify(sss, kv, batch=0) == 0
    for st in range(5):
        assert lib.sss_status_string(st).startswith(b"SSS_")


# --------------------------------------------------------------------------
# fused step: struct layout and host-side validation (nothing is launched)
# --------------------------------------------------------------------------
LAYOUT_C = r'''
#include <stddef.h>
#include <stdio.h>
#include "sss.h"
#define F(T, f) printf(#T " " #f " %zu\n", offsetof(T, f));
int main(void) {
  printf("sss_paged_kv size %zu\n", sizeof(sss_paged_kv));
  printf("sss_verify_step size %zu\n", sizeof(sss_verify_step));
  printf("sss_draft_step size %zu\n", sizeof(sss_draft_step));
  F(sss_paged_kv, k) F(sss_paged_kv, v) F(sss_paged_kv, dtype) F(sss_paged_kv, num_pages)
  F(sss_paged_kv, page_size) F(sss_paged_kv, num_kv_heads) F(sss_paged_kv, head_dim)
  F(sss_paged_kv, max_pages_per_req) F(sss_paged_kv, page_table) F(sss_paged_kv, seq_lens)
  F(sss_paged_kv, max_seq_len)
  F(sss_verify_step, kv) F(sss_verify_step, q) F(sss_verify_step, batch) F(sss_verify_step, n_q)
  F(sss_verify_step, num_q_heads) F(sss_verify_step, sm_scale) F(sss_verify_step, block_size)
  F(sss_verify_step, score_row_start) F(sss_verify_step, max_blocks) F(sss_verify_step, o)
  F(sss_verify_step, lse) F(sss_verify_step, block_scores) F(sss_verify_step, budget)
  F(sss_verify_step, window) F(sss_verify_step, sel) F(sss_verify_step, sel_count)
  F(sss_verify_step, max_sel)
  F(sss_draft_step, kv) F(sss_draft_step, q) F(sss_draft_step, batch) F(sss_draft_step, num_q_heads)
  F(sss_draft_step, sm_scale) F(sss_draft_step, block_size) F(sss_draft_step, sel)
  F(sss_draft_step, sel_count) F(sss_draft_step, max_sel) F(sss_draft_step, window)
  F(sss_draft_step, o) F(sss_draft_step, lse)
  return 0;
}
'''


def test_struct_layout_matches_header(tmp_path):
    """The binding's ctypes structures have the C header's field offsets."""
    import shutil
    import subprocess
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    src = tmp_path / "layout.c"
    exe = tmp_path / "layout"
    src.write_text(LAYOUT_C)
    subprocess.run(["gcc", "-I", os.path.dirname(HDR), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    sss = _binding()
    types = {"sss_paged_kv": sss.PagedKV, "sss_verify_step": sss.VerifyStep,
             "sss_draft_step": sss.DraftStep}
    for line in out.splitlines():
        t, f, n = line.split()
        if f == "size":
            assert ctypes.sizeof(types[t]) == int(n), line
        else:
            assert getattr(types[t], f).offset == int(n), line


def fused_args(sss, vkw=None, dkw=None, kvkw=None):
    kv = good_kv(sss, **(kvkw or {}))
    v = dict(kv=kv, q=4096, batch=2, n_q=5, num_q_heads=8, sm_scale=0.1, block_size=16,
             score_row_start=0, max_blocks=8, o=8192, lse=16384, block_scores=32768, budget=256,
             window=64, sel=1 << 20, sel_count=1 << 21, max_sel=4)
    v.update(vkw or {})
    d = dict(kv=kv, q=12288, batch=2, num_q_heads=8, sm_scale=0.1, block_size=16, sel=1 << 20,
             sel_count=1 << 21, max_sel=4, window=64, o=20480, lse=24576)
    d.update(dkw or {})
    return sss.VerifyStep(**v), sss.DraftStep(**d)


def call_fused(sss, v, d, chained, wsb=1 << 30):
    return sss.raw().sss_fused_step(None if v is None else ctypes.byref(v),
                                    None if d is None else ctypes.byref(d), chained, 1 << 22, wsb,
                                    None)


@pytest.mark.parametrize("vkw,dkw,kvkw,chained,status", [
    ({}, dict(sel=1 << 23), {}, 1, 1),                  # chained draft must read verify's selection
    ({}, dict(batch=1), {}, 1, 1),                      # chained batches differ
    ({}, dict(max_sel=3), {}, 1, 1),
    (dict(sel=None), {}, {}, 1, 1),                     # chained step needs a selection
    ({}, {}, {}, 0, 1),                                 # unchained: output aliases input
    ({}, {}, dict(dtype=0), 0, 2),                      # fp32 cache: no matrix-core path
    (dict(n_q=0), {}, {}, 0, 1),
    (dict(window=-1), dict(sel=1 << 23, sel_count=1 << 24), {}, 0, 1),
    ({}, dict(sel=1 << 23, sel_count=1 << 24, num_q_heads=2 * 64), {}, 0, 2),   # draft G = 64
])
def test_fused_rejects_bad_arguments(vkw, dkw, kvkw, chained, status):
    sss = _binding()
    v, d = fused_args(sss, vkw, dkw, kvkw)
    assert call_fused(sss, v, d, chained) == status
    assert sss.raw().sss_last_error()


def test_fused_rows_split_form():
    """Chained steps of split 65-96-row units (fewer than 1024) take the
    rows-split form; its workspace covers the verify and draft partials."""
    sss = _binding()

    def form(batch, L, n_q=5, hq=32, chained=True):
        kv = dict(num_kv_heads=2, max_seq_len=L, max_pages_per_req=-(-L // 64),
                  num_pages=batch * -(-L // 64), page_size=64)
        nblk = -(-L // 64)
        v, d = fused_args(sss, dict(batch=batch, num_q_heads=hq, n_q=n_q, block_size=64,
                                    max_blocks=nblk, max_sel=16, window=128),
                          dict(batch=batch, num_q_heads=hq, block_size=64, max_sel=16,
                               window=128), kv)
        if not chained:
            d.sel, d.sel_count = 1 << 23, 1 << 24
        return sss.fused_step_form(v, d, chained), sss.fused_workspace_size(v, d, chained)

    f, ws = form(4, 131072)                       # 8 units x 64 chunks of 80 rows
    assert f == "rows_split"
    # verify partials (fp32 O and LSE) and block masses dominate the workspace
    assert ws >= 8 * 64 * 80 * (128 + 1) * 4 + 8 * 2048 * 80 * 4
    assert form(2, 3000)[0] == "rows_split"
    assert form(2, 3000, n_q=6)[0] == "rows_split"  # 96 rows
    assert form(1, 2000)[0] == "rows_split"        # 10 draft chunks, 8 verify chunks
    assert form(2, 3000, n_q=2)[0] == "work_list"  # 32 rows: one row tile
    assert form(4, 131072, chained=False)[0] == "work_list"


def test_fused_workspace_query_and_size_check():
    sss = _binding()
    # short requests: every unit fits in one chunk, nothing to stage
    v, d = fused_args(sss)
    assert sss.fused_workspace_size(v, d, True) == 0
    # long requests: units split, partials and block masses are staged
    long_kv = dict(max_seq_len=8192, max_pages_per_req=512)
    v, d = fused_args(sss, vkw=dict(max_blocks=512), kvkw=long_kv)
    n = sss.fused_workspace_size(v, d, True)
    assert n > 0 and n % 256 == 0
    assert call_fused(sss, v, d, 1, wsb=n - 1) == 3
    v2, d2 = fused_args(sss, vkw=dict(max_blocks=512), dkw=dict(sel=1 << 23, sel_count=1 << 24),
                        kvkw=long_kv)
    assert sss.fused_workspace_size(v2, d2, False) > 0
    d3 = fused_args(sss, dkw=dict(max_sel=600), kvkw=long_kv)[1]
    assert sss.fused_workspace_size(None, d3, False) > 0
    # nothing to do: a successful no-op
    assert call_fused(sss, None, None, 0) == 0
    v0, d0 = fused_args(sss, vkw=dict(batch=0), dkw=dict(batch=0))
    assert call_fused(sss, v0, d0, 0) == 0


def test_kv_update_rejects_bad_arguments():
    sss = _binding()
    lib = sss.raw()
    kv = good_kv(sss)
    w = lib.sss_kv_write
    assert w(ctypes.byref(kv), 4096, 8192, -1, 2, 256, None) == 1
    assert w(ctypes.byref(kv), 4096, 8192, 2, -1, 256, None) == 1
    assert w(ctypes.byref(kv), 4100, 8192, 2, 2, 256, None) == 1      # misaligned rows
    assert w(ctypes.byref(kv), None, 8192, 2, 2, 256, None) == 1
    assert w(ctypes.byref(good_kv(sss, head_dim=96)), 4096, 8192, 2, 2, 256, None) == 2
    assert w(ctypes.byref(kv), 4096, 8192, 2, 0, 256, None) == 0      # nothing to write
    c = lib.sss_kv_commit
    assert c(256, 512, 2, 0, 256, None) == 1
    assert c(256, 512, -1, 5, 256, None) == 1
    assert c(None, 512, 2, 5, 256, None) == 1
    assert c(256, 512, 0, 5, 256, None) == 0


def call_sparse(sss, kv, **kw):
    a = dict(q=4096, batch=2, n_q=5, hq=8, scale=0.1, bs=16, rsel=256, rcnt=512, max_sel=4,
             window=16, splits=0, o=8192, lse=16384, ws=65536, wsb=1 << 30)
    a.update(kw)
    return sss.raw().sss_sparse_verify_attn(ctypes.byref(kv), a["q"], a["batch"], a["n_q"],
                                            a["hq"], a["scale"], a["bs"], a["rsel"], a["rcnt"],
                                            a["max_sel"], a["window"], a["splits"], a["o"],
                                            a["lse"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kvkw,callkw,status", [
    (dict(dtype=0), {}, 2),                      # fp32 cache: matrix-core path only
    (dict(page_size=8, max_pages_per_req=16), {}, 2),
    ({}, dict(bs=8), 2),
    ({}, dict(n_q=0), 1),
    ({}, dict(n_q=33), 1),
    ({}, dict(hq=7), 1),
    ({}, dict(hq=128, n_q=5), 2),                # 5 * 64 rows > 128
    ({}, dict(max_sel=0), 1),
    ({}, dict(window=-1), 1),
    ({}, dict(splits=-1), 1),
    ({}, dict(scale=float("inf")), 1),
    ({}, dict(q=4100), 1),
    ({}, dict(o=0), 1),
    ({}, dict(rsel=0), 1),
    ({}, dict(rcnt=514), 1),                     # misaligned counts
    (dict(max_seq_len=1024, max_pages_per_req=64), dict(wsb=16, splits=4), 3),
    (dict(max_seq_len=1024, max_pages_per_req=64), dict(ws=65537, splits=4), 1),
])
def test_sparse_verify_rejects_bad_arguments(kvkw, callkw, status):
    sss = _binding()
    kv = good_kv(sss, **kvkw)
    assert call_sparse(sss, kv, **callkw) == status
    assert sss.raw().sss_last_error()


def test_sparse_verify_workspace_and_empty_batch():
    sss = _binding()
    kv = good_kv(sss)
    assert call_sparse(sss, kv, batch=0) == 0
    assert sss.sparse_verify_workspace_size(kv, 2, 5, 8, 16, 4, 16, 1) == 0   # one chunk
    long_kv = good_kv(sss, max_seq_len=1024, max_pages_per_req=64)
    n = sss.sparse_verify_workspace_size(long_kv, 2, 5, 8, 16, 40, 16, 4)
    assert n > 0 and n % 256 == 0
    with pytest.raises(sss.SSSError):
        sss.sparse_verify_workspace_size(good_kv(sss, dtype=0), 2, 5, 8, 16, 4, 16, 0)


def test_pool_of_2_31_rows_is_unsupported():
    sss = _binding()
    kv = good_kv(sss, num_pages=1 << 26, page_size=16, num_kv_heads=2)   # 2^31 rows
    assert call_verify(sss, kv) == 2
    assert b"2^31" in sss.raw().sss_last_error()


def test_binding_refuses_host_and_strided_tensors():
    """The library reads plain device pointers: the binding refuses host
    tensors, strided views and wrong index dtypes before any call."""
    import torch
    sss = _binding()
    k = torch.zeros((4, 2, 16, 64), dtype=torch.bfloat16)
    table = torch.zeros((1, 4), dtype=torch.int32)
    lens = torch.ones((1,), dtype=torch.int32)
    with pytest.raises(ValueError):
        sss.paged_kv(k, k, table, lens, 64)                      # host memory
    with pytest.raises(TypeError):
        sss.paged_kv(k, k, table.long(), lens, 64)                # int64 page table
    with pytest.raises(ValueError):
        sss._ptr(torch.zeros((4, 4))[:, ::2])


def test_binding_checks_shapes_against_the_cache():
    """Sizes cannot be checked below the C ABI (plain pointers): the binding
    compares every buffer with the cache description before any call."""
    import torch
    sss = _binding()
    kv = good_kv(sss)                                   # bf16, Hkv 2, d 128
    kv._batch = 2
    q = torch.zeros((2, 5, 8, 128), dtype=torch.bfloat16)
    lse = torch.zeros((2, 5, 8))
    sc = torch.zeros((2, 2, 8))
    with pytest.raises(ValueError):                     # head_dim 64 against 128
        sss.verify_attn(kv, q[..., :64].contiguous(), 0.1, 16, 8, q[..., :64].contiguous(), lse, sc)
    with pytest.raises(TypeError):                      # fp32 queries on a bf16 cache
        sss.verify_attn(kv, q.float(), 0.1, 16, 8, q.float(), lse, sc)
    with pytest.raises(ValueError):                     # more requests than the table holds
        q3 = torch.zeros((3, 5, 8, 128), dtype=torch.bfloat16)
        sss.verify_attn(kv, q3, 0.1, 16, 8, q3, torch.zeros((3, 5, 8)), torch.zeros((3, 2, 8)))
    with pytest.raises(ValueError):                     # block scores too short
        sss.verify_attn(kv, q, 0.1, 16, 8, q, lse, sc[..., :4].contiguous())
    sel = torch.zeros((2, 2, 4), dtype=torch.int32)
    with pytest.raises(ValueError):                     # sel_count of another shape
        sss.block_topk(sc, torch.ones(2, dtype=torch.int32), 16,
                       torch.ones(2, dtype=torch.int32), 0, sel, torch.zeros(2, dtype=torch.int32))
    with pytest.raises(ValueError):                     # new rows of another head count
        sss.kv_write(kv, torch.zeros((2, 5, 4, 128), dtype=torch.bfloat16),
                     torch.zeros((2, 5, 4, 128), dtype=torch.bfloat16),
                     torch.zeros(2, dtype=torch.int32))


def test_noalloc_verify_checks_on_the_host():
    """sss_verify_attn_noalloc validates like sss_verify_attn and refuses,
    before touching the device, a call whose workspace exceeds its static
    scratch (the size the binding and the header state)."""
    sss = _binding()
    lib = sss.raw()
    hdr = open(HDR).read()
    assert re.search(r"#define SSS_NOALLOC_SCRATCH_BYTES \(\(size_t\)32 << 20\)", hdr)
    assert sss.NOALLOC_SCRATCH_BYTES == 32 << 20
    kv = good_kv(sss)
    f = lib.sss_verify_attn_noalloc
    assert f(ctypes.byref(kv), 4096, 2, 0, 8, 0.1, 16, 0, 0, 8192, 16384, 32768, 8, None) == 1
    assert f(ctypes.byref(kv), 4096, 2, 5, 7, 0.1, 16, 0, 0, 8192, 16384, 32768, 8, None) == 1
    assert f(ctypes.byref(good_kv(sss, head_dim=96)), 4096, 2, 5, 8, 0.1, 16, 0, 0, 8192, 16384,
             32768, 8, None) == 2
    assert f(ctypes.byref(kv), 4096, 0, 5, 8, 0.1, 16, 0, 0, 8192, 16384, 32768, 8, None) == 0
    big = sss.PagedKV(k=256, v=512, dtype=sss.SSS_BF16, num_pages=16384, page_size=64,
                      num_kv_heads=2, head_dim=128, max_pages_per_req=2048, page_table=1024,
                      seq_lens=2048, max_seq_len=131072)
    assert sss.verify_workspace_size(big, 8, 5, 32, 64, 2048, 64) > sss.NOALLOC_SCRATCH_BYTES
    assert f(ctypes.byref(big), 4096, 8, 5, 32, 0.088, 64, 0, 64, 8192, 16384, 32768, 2048,
             None) == 3
    assert b"needs" in lib.sss_last_error() or b"need" in lib.sss_last_error()


def test_probes_reject_bad_arguments():
    sss = _binding()
    lib = sss.raw()
    lib.sss_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                          ctypes.c_void_p]
    lib.sss_probe_paged_read.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                         ctypes.c_void_p]
    assert lib.sss_probe_stream_read(None, 16, 256, None) == 1
    assert lib.sss_probe_stream_read(264, 16, 256, None) == 1      # misaligned source
    assert lib.sss_probe_stream_read(256, 17, 256, None) == 1      # not a multiple of 16 bytes
    assert lib.sss_probe_stream_read(256, 0, 256, None) == 0       # nothing to read
    kv = good_kv(sss)
    assert lib.sss_probe_paged_read(ctypes.addressof(kv), -1, 256, None) == 1
    assert lib.sss_probe_paged_read(ctypes.addressof(kv), 2, None, None) == 1
    assert lib.sss_probe_paged_read(ctypes.addressof(good_kv(sss, dtype=7)), 2, 256, None) == 2
    assert lib.sss_probe_paged_read(ctypes.addressof(good_kv(sss, page_size=1, head_dim=1)), 2,
                                    256, None) == 2                 # 2-byte runs
    assert lib.sss_probe_paged_read(ctypes.addressof(kv), 0, 256, None) == 0


def test_fused_step_form():
    """The launch form sss_fused_step takes (host query, nothing launched):
    chained decode steps of >= 512 whole units whose verify runs two
    workgroups per compute unit are persistent, unless there are >= 1024
    units of <= 1024 candidates (then one wave per unit selects and drafts
    after the verify launch: two launches)."""
    sss = _binding()

    def form(batch, L, chained=True, **vkw):
        kv = dict(num_kv_heads=8, max_seq_len=L, max_pages_per_req=-(-L // 16),
                  num_pages=batch * -(-L // 16))
        nblk = -(-L // 16)
        v, d = fused_args(sss, dict(batch=batch, num_q_heads=32, max_blocks=nblk, max_sel=26,
                                    **vkw),
                          dict(batch=batch, num_q_heads=32, max_sel=26), kv)
        if not chained:
            d.sel, d.sel_count = 1 << 23, 1 << 24
        return sss.fused_step_form(v, d, chained)

    assert form(128, 8192) == "two_launch"         # the batch-128 x 8K decode step
    assert form(64, 8192) == "persistent"          # 512 units
    assert form(96, 1500) == "persistent"          # 768 units
    assert form(128, 1500) == "two_launch"
    assert form(128, 16384) == "two_launch"        # 1024 candidates per unit
    assert form(63, 8192) == "work_list"           # 504 units: split to fill the GPU
    assert form(128, 512) == "two_launch"          # four-group verify fits twice per CU
    assert form(128, 8192, chained=False) == "work_list"
    assert form(16, 4096) == "work_list"
    v, d = fused_args(sss)
    assert sss.fused_step_form(None, None, False) == "nothing"
    with pytest.raises(sss.SSSError):
        sss.fused_step_form(v, None, True)         # chained without a draft half
