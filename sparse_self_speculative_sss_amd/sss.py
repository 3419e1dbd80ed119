"""Thin ctypes binding of libsss.so (C ABI in include/sss.h).

Each function marshals torch tensors into the C call with the same name and
launches on ``torch.cuda.current_stream()``.  All arithmetic runs in the HIP
library; if it is missing this module raises on import.  Workspaces are
allocated here as plain device byte tensors (the library never allocates).
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsss.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(
        f"{_LIB_PATH} is missing: build it with `python -m sparse_self_speculative_sss_amd.build`")
_lib = ctypes.CDLL(_LIB_PATH)

SSS_OK, SSS_ERR_INVALID_ARGUMENT, SSS_ERR_UNSUPPORTED, SSS_ERR_WORKSPACE_TOO_SMALL, SSS_ERR_HIP = range(5)
SSS_F32, SSS_BF16 = 0, 1
# size of the static device scratch of sss_verify_attn_noalloc (SSS_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 32 << 20

_c_int = ctypes.c_int32
_vp = ctypes.c_void_p
_fp = ctypes.c_void_p


class PagedKV(ctypes.Structure):
    _fields_ = [
        ("k", _vp), ("v", _vp), ("dtype", _c_int), ("num_pages", _c_int),
        ("page_size", _c_int), ("num_kv_heads", _c_int), ("head_dim", _c_int),
        ("max_pages_per_req", _c_int), ("page_table", _vp), ("seq_lens", _vp),
        ("max_seq_len", _c_int),
    ]


_lib.sss_verify_attn.restype = _c_int
_lib.sss_verify_attn.argtypes = [ctypes.POINTER(PagedKV), _vp, _c_int, _c_int, _c_int,
                                 ctypes.c_float, _c_int, _c_int, _c_int, _vp, _fp, _fp, _c_int,
                                 _vp, ctypes.c_size_t, _vp]
_lib.sss_verify_workspace_size.restype = ctypes.c_size_t
_lib.sss_verify_workspace_size.argtypes = [ctypes.POINTER(PagedKV), _c_int, _c_int, _c_int,
                                           _c_int, _c_int, _c_int]
_lib.sss_verify_attn_noalloc.restype = _c_int
_lib.sss_verify_attn_noalloc.argtypes = [ctypes.POINTER(PagedKV), _vp, _c_int, _c_int, _c_int,
                                         ctypes.c_float, _c_int, _c_int, _c_int, _vp, _fp, _fp,
                                         _c_int, _vp]
_lib.sss_block_topk.restype = _c_int
_lib.sss_block_topk.argtypes = [_fp, _c_int, _c_int, _c_int, _vp, _c_int, _vp, _c_int, _vp, _vp,
                                _c_int, _vp]
_lib.sss_draft_attn.restype = _c_int
_lib.sss_draft_attn.argtypes = [ctypes.POINTER(PagedKV), _vp, _c_int, _c_int, ctypes.c_float,
                                _c_int, _vp, _vp, _c_int, _c_int, _c_int, _vp, _fp, _vp,
                                ctypes.c_size_t, _vp]
_lib.sss_draft_workspace_size.restype = ctypes.c_size_t
_lib.sss_draft_workspace_size.argtypes = [ctypes.POINTER(PagedKV), _c_int, _c_int, _c_int, _c_int,
                                          _c_int, _c_int]
_lib.sss_sparse_verify_attn.restype = _c_int
_lib.sss_sparse_verify_attn.argtypes = [ctypes.POINTER(PagedKV), _vp, _c_int, _c_int, _c_int,
                                        ctypes.c_float, _c_int, _vp, _vp, _c_int, _c_int, _c_int,
                                        _vp, _fp, _vp, ctypes.c_size_t, _vp]
_lib.sss_sparse_verify_workspace_size.restype = ctypes.c_size_t
_lib.sss_sparse_verify_workspace_size.argtypes = [ctypes.POINTER(PagedKV), _c_int, _c_int, _c_int,
                                                  _c_int, _c_int, _c_int, _c_int]
_lib.sss_merge.restype = _c_int
_lib.sss_merge.argtypes = [_fp, _fp, _c_int, _c_int, _c_int, _vp, _c_int, _fp, _vp]


class VerifyStep(ctypes.Structure):
    """sss_verify_step (include/sss.h)."""
    _fields_ = [
        ("kv", PagedKV), ("q", _vp), ("batch", _c_int), ("n_q", _c_int), ("num_q_heads", _c_int),
        ("sm_scale", ctypes.c_float), ("block_size", _c_int), ("score_row_start", _c_int),
        ("max_blocks", _c_int), ("o", _vp), ("lse", _vp), ("block_scores", _vp), ("budget", _vp),
        ("window", _c_int), ("sel", _vp), ("sel_count", _vp), ("max_sel", _c_int),
    ]


class DraftStep(ctypes.Structure):
    """sss_draft_step (include/sss.h)."""
    _fields_ = [
        ("kv", PagedKV), ("q", _vp), ("batch", _c_int), ("num_q_heads", _c_int),
        ("sm_scale", ctypes.c_float), ("block_size", _c_int), ("sel", _vp), ("sel_count", _vp),
        ("max_sel", _c_int), ("window", _c_int), ("o", _vp), ("lse", _vp),
    ]


_lib.sss_fused_step.restype = _c_int
_lib.sss_fused_step.argtypes = [ctypes.POINTER(VerifyStep), ctypes.POINTER(DraftStep), _c_int,
                                _vp, ctypes.c_size_t, _vp]
_lib.sss_fused_step_marked.restype = _c_int
_lib.sss_fused_step_marked.argtypes = [ctypes.POINTER(VerifyStep), ctypes.POINTER(DraftStep),
                                       _c_int, _vp, ctypes.c_size_t, _vp, _vp]
_lib.sss_fused_step_form.restype = _c_int
_lib.sss_fused_step_form.argtypes = [ctypes.POINTER(VerifyStep), ctypes.POINTER(DraftStep), _c_int]
_lib.sss_fused_workspace_size.restype = ctypes.c_size_t
_lib.sss_fused_workspace_size.argtypes = [ctypes.POINTER(VerifyStep), ctypes.POINTER(DraftStep),
                                          _c_int]
_lib.sss_kv_write.restype = _c_int
_lib.sss_kv_write.argtypes = [ctypes.POINTER(PagedKV), _vp, _vp, _c_int, _c_int, _vp, _vp]
_lib.sss_kv_commit.restype = _c_int
_lib.sss_kv_commit.argtypes = [_vp, _vp, _c_int, _c_int, _vp, _vp]
_lib.sss_status_string.restype = ctypes.c_char_p
_lib.sss_status_string.argtypes = [_c_int]
_lib.sss_last_error.restype = ctypes.c_char_p
_lib.sss_last_error.argtypes = []
_lib.sss_version.restype = _c_int
_lib.sss_version.argtypes = []

EXPORTED = ["sss_verify_attn", "sss_verify_workspace_size", "sss_verify_attn_noalloc",
            "sss_block_topk", "sss_draft_attn", "sss_draft_workspace_size", "sss_merge",
            "sss_fused_step", "sss_fused_step_marked", "sss_fused_workspace_size",
            "sss_fused_step_form",
            "sss_kv_write", "sss_kv_commit", "sss_sparse_verify_attn",
            "sss_sparse_verify_workspace_size", "sss_status_string", "sss_last_error",
            "sss_version"]


class SSSError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.sss_last_error().decode()
        super().__init__(f"{where}: {_lib.sss_status_string(status).decode()}: {msg}")


def _check(status: int, where: str):
    if status != SSS_OK:
        raise SSSError(status, where)


def _ptr(t):
    """Device address of a tensor.  The library reads plain pointers, so a
    host or strided tensor is refused here rather than handed to a kernel."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"expected a device tensor, got one on {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"expected a contiguous tensor (shape {tuple(t.shape)}, "
                         f"strides {t.stride()})")
    return ctypes.c_void_p(t.data_ptr())


def _addr(t):
    """_ptr as a plain integer (for the step structs)."""
    return None if t is None else _ptr(t).value


_TORCH_DTYPE = {SSS_F32: torch.float32, SSS_BF16: torch.bfloat16}


def _expect(t, shape, what, dtype=None):
    """Buffer sizes cannot be checked by the library (plain pointers): a
    tensor of another shape would be read or written out of bounds."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{what}: dtype {t.dtype}, expected {dtype}")


def _requests(kv, B, what):
    """The batch of a call may not exceed the requests kv describes."""
    n = getattr(kv, "_batch", None)
    if n is not None and B > n:
        raise ValueError(f"{what}: batch {B} exceeds the {n} requests of the paged cache")


def _i32(t, what):
    if t is not None and t.dtype != torch.int32:
        raise TypeError(f"{what} must be int32, got {t.dtype}")
    return t


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SSS_F32
    if t.dtype == torch.bfloat16:
        return SSS_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def paged_kv(k_cache, v_cache, page_table, seq_lens, max_seq_len: int) -> PagedKV:
    """Describe a paged cache [num_pages][Hkv][page_size][d] to the library."""
    if k_cache.dtype != v_cache.dtype or k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must have the same dtype and shape")
    _i32(page_table, "page_table")
    _i32(seq_lens, "seq_lens")
    for t in (k_cache, v_cache, page_table, seq_lens):
        _ptr(t)
    if page_table.dim() != 2 or tuple(seq_lens.shape) != (page_table.shape[0],):
        raise ValueError("page_table must be [batch][max_pages] and seq_lens [batch]")
    kv = PagedKV(k=k_cache.data_ptr(), v=v_cache.data_ptr(), dtype=_dtype_code(k_cache),
                 num_pages=k_cache.shape[0], page_size=k_cache.shape[2],
                 num_kv_heads=k_cache.shape[1], head_dim=k_cache.shape[3],
                 max_pages_per_req=page_table.shape[1], page_table=page_table.data_ptr(),
                 seq_lens=seq_lens.data_ptr(), max_seq_len=int(max_seq_len))
    kv._batch = int(page_table.shape[0])
    return kv


def verify_workspace_size(kv: PagedKV, batch, n_q, num_q_heads, block_size, max_blocks,
                          num_splits=0) -> int:
    n = _lib.sss_verify_workspace_size(ctypes.byref(kv), batch, n_q, num_q_heads, block_size,
                                       max_blocks, num_splits)
    if n == 0 and _lib.sss_last_error():
        raise SSSError(SSS_ERR_INVALID_ARGUMENT, "sss_verify_workspace_size")
    return n


def draft_workspace_size(kv: PagedKV, batch, num_q_heads, block_size, max_sel, window,
                         num_splits=0) -> int:
    n = _lib.sss_draft_workspace_size(ctypes.byref(kv), batch, num_q_heads, block_size, max_sel,
                                      window, num_splits)
    if n == 0 and _lib.sss_last_error():
        raise SSSError(SSS_ERR_INVALID_ARGUMENT, "sss_draft_workspace_size")
    return n


def sparse_verify_workspace_size(kv: PagedKV, batch, n_q, num_q_heads, block_size, max_sel,
                                 window, num_splits=0) -> int:
    n = _lib.sss_sparse_verify_workspace_size(ctypes.byref(kv), batch, n_q, num_q_heads,
                                              block_size, max_sel, window, num_splits)
    if n == 0 and _lib.sss_last_error():
        raise SSSError(SSS_ERR_INVALID_ARGUMENT, "sss_sparse_verify_workspace_size")
    return n


def workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def verify_attn(kv: PagedKV, q, sm_scale, block_size, max_blocks, o, lse, block_scores,
                ws=None, score_row_start=0, num_splits=0):
    """sss_verify_attn on tensors: q/o [B][n_q][Hq][d], lse [B][n_q][Hq],
    block_scores [B][Hkv][max_blocks]."""
    B, n_q, hq, _ = q.shape
    _requests(kv, B, "verify_attn")
    _expect(q, (B, n_q, hq, kv.head_dim), "q", _TORCH_DTYPE.get(kv.dtype))
    _expect(o, q.shape, "o", q.dtype)
    _expect(lse, (B, n_q, hq), "lse", torch.float32)
    _expect(block_scores, (B, kv.num_kv_heads, max_blocks), "block_scores", torch.float32)
    if ws is None:
        ws = workspace(verify_workspace_size(kv, B, n_q, hq, block_size, max_blocks, num_splits),
                       q.device)
    _check(_lib.sss_verify_attn(ctypes.byref(kv), _ptr(q), B, n_q, hq, float(sm_scale), block_size,
                                score_row_start, num_splits, _ptr(o), _ptr(lse),
                                _ptr(block_scores), max_blocks, _ptr(ws), ws.numel(), _stream()),
           "sss_verify_attn")
    return o, lse, block_scores


def verify_attn_noalloc(kv: PagedKV, q, sm_scale, block_size, max_blocks, o, lse, block_scores,
                        score_row_start=0, num_splits=0):
    """sss_verify_attn_noalloc: verify_attn with the library's static device
    scratch instead of a workspace (no allocation on either side)."""
    B, n_q, hq, _ = q.shape
    _requests(kv, B, "verify_attn_noalloc")
    _expect(q, (B, n_q, hq, kv.head_dim), "q", _TORCH_DTYPE.get(kv.dtype))
    _expect(o, q.shape, "o", q.dtype)
    _expect(lse, (B, n_q, hq), "lse", torch.float32)
    _expect(block_scores, (B, kv.num_kv_heads, max_blocks), "block_scores", torch.float32)
    _check(_lib.sss_verify_attn_noalloc(ctypes.byref(kv), _ptr(q), B, n_q, hq, float(sm_scale),
                                        block_size, score_row_start, num_splits, _ptr(o),
                                        _ptr(lse), _ptr(block_scores), max_blocks, _stream()),
           "sss_verify_attn_noalloc")
    return o, lse, block_scores


def sparse_verify_attn(kv: PagedKV, q, sm_scale, block_size, row_sel, row_sel_count, window, o,
                       lse, ws=None, num_splits=0):
    """sss_sparse_verify_attn: q/o [B][n_q][Hq][d], lse [B][n_q][Hq],
    row_sel [B][Hkv][n_q][max_sel], row_sel_count [B][Hkv][n_q]."""
    B, n_q, hq, _ = q.shape
    max_sel = row_sel.shape[3]
    _requests(kv, B, "sparse_verify_attn")
    _expect(q, (B, n_q, hq, kv.head_dim), "q", _TORCH_DTYPE.get(kv.dtype))
    _expect(o, q.shape, "o", q.dtype)
    _expect(lse, (B, n_q, hq), "lse", torch.float32)
    _expect(row_sel, (B, kv.num_kv_heads, n_q, max_sel), "row_sel", torch.int32)
    _expect(row_sel_count, (B, kv.num_kv_heads, n_q), "row_sel_count", torch.int32)
    if ws is None:
        ws = workspace(sparse_verify_workspace_size(kv, B, n_q, hq, block_size, max_sel, window,
                                                    num_splits), q.device)
    _check(_lib.sss_sparse_verify_attn(ctypes.byref(kv), _ptr(q), B, n_q, hq, float(sm_scale),
                                       block_size, _ptr(row_sel), _ptr(row_sel_count), max_sel,
                                       window, num_splits, _ptr(o), _ptr(lse), _ptr(ws),
                                       ws.numel(), _stream()),
           "sss_sparse_verify_attn")
    return o, lse


def block_topk(block_scores, seq_lens, block_size, budget, window, sel, sel_count):
    """sss_block_topk: sel [B][Hkv][max_sel], sel_count [B][Hkv]."""
    B, hkv, max_blocks = block_scores.shape
    _expect(block_scores, (B, hkv, max_blocks), "block_scores", torch.float32)
    _expect(seq_lens, (B,), "seq_lens", torch.int32)
    _expect(budget, (B,), "budget", torch.int32)
    _expect(sel, (B, hkv, sel.shape[2]), "sel", torch.int32)
    _expect(sel_count, (B, hkv), "sel_count", torch.int32)
    _check(_lib.sss_block_topk(_ptr(block_scores), B, hkv, max_blocks, _ptr(seq_lens), block_size,
                               _ptr(budget), window, _ptr(sel), _ptr(sel_count), sel.shape[2],
                               _stream()),
           "sss_block_topk")
    return sel, sel_count


def draft_attn(kv: PagedKV, q, sm_scale, block_size, sel, sel_count, window, o, lse, ws=None,
               num_splits=0):
    """sss_draft_attn: q/o [B][1][Hq][d], lse [B][1][Hq]."""
    B, _, hq, _ = q.shape
    max_sel = sel.shape[2]
    _requests(kv, B, "draft_attn")
    _expect(q, (B, 1, hq, kv.head_dim), "q", _TORCH_DTYPE.get(kv.dtype))
    _expect(o, q.shape, "o", q.dtype)
    _expect(lse, (B, 1, hq), "lse", torch.float32)
    _expect(sel, (B, kv.num_kv_heads, max_sel), "sel", torch.int32)
    _expect(sel_count, (B, kv.num_kv_heads), "sel_count", torch.int32)
    if ws is None:
        ws = workspace(draft_workspace_size(kv, B, hq, block_size, max_sel, window, num_splits),
                       q.device)
    _check(_lib.sss_draft_attn(ctypes.byref(kv), _ptr(q), B, hq, float(sm_scale), block_size,
                               _ptr(sel), _ptr(sel_count), max_sel, window, num_splits, _ptr(o),
                               _ptr(lse), _ptr(ws), ws.numel(), _stream()),
           "sss_draft_attn")
    return o, lse


def merge(o_parts, lse_parts, o, lse=None):
    """sss_merge: o_parts [S][rows][d] fp32, lse_parts [S][rows] -> o [rows][d]."""
    S, rows, d = o_parts.shape
    _expect(o_parts, (S, rows, d), "o_parts", torch.float32)
    _expect(lse_parts, (S, rows), "lse_parts", torch.float32)
    _expect(o, (rows, d), "o")
    _expect(lse, (rows,), "lse", torch.float32)
    _check(_lib.sss_merge(_ptr(o_parts), _ptr(lse_parts), S, rows, d, _ptr(o), _dtype_code(o),
                          _ptr(lse), _stream()),
           "sss_merge")
    return o, lse


def verify_step(kv: PagedKV, q, sm_scale, block_size, max_blocks, o, lse, block_scores,
                score_row_start=0, budget=None, window=0, sel=None, sel_count=None) -> VerifyStep:
    """Verify half of a fused step (tensors as for verify_attn; with sel /
    sel_count / budget, the step also selects, as block_topk does)."""
    B, n_q, hq, _ = q.shape
    _requests(kv, B, "verify_step")
    _expect(q, (B, n_q, hq, kv.head_dim), "q", _TORCH_DTYPE.get(kv.dtype))
    _expect(o, q.shape, "o", q.dtype)
    _expect(lse, (B, n_q, hq), "lse", torch.float32)
    _expect(block_scores, (B, kv.num_kv_heads, max_blocks), "block_scores", torch.float32)
    _expect(budget, (B,), "budget", torch.int32)
    if sel is not None:
        _expect(sel, (B, kv.num_kv_heads, sel.shape[2]), "sel", torch.int32)
    _expect(sel_count, (B, kv.num_kv_heads), "sel_count", torch.int32)
    return VerifyStep(kv=kv, q=_addr(q), batch=B, n_q=n_q, num_q_heads=hq,
                      sm_scale=float(sm_scale), block_size=block_size,
                      score_row_start=score_row_start, max_blocks=max_blocks, o=_addr(o),
                      lse=_addr(lse), block_scores=_addr(block_scores),
                      budget=_addr(budget), window=int(window),
                      sel=_addr(sel),
                      sel_count=_addr(sel_count),
                      max_sel=0 if sel is None else sel.shape[2])


def draft_step(kv: PagedKV, q, sm_scale, block_size, sel, sel_count, window, o, lse) -> DraftStep:
    """Draft half of a fused step (tensors as for draft_attn)."""
    B, _, hq, _ = q.shape
    _requests(kv, B, "draft_step")
    _expect(q, (B, 1, hq, kv.head_dim), "q", _TORCH_DTYPE.get(kv.dtype))
    _expect(o, q.shape, "o", q.dtype)
    _expect(lse, (B, 1, hq), "lse", torch.float32)
    _expect(sel, (B, kv.num_kv_heads, sel.shape[2]), "sel", torch.int32)
    _expect(sel_count, (B, kv.num_kv_heads), "sel_count", torch.int32)
    return DraftStep(kv=kv, q=_addr(q), batch=B, num_q_heads=hq, sm_scale=float(sm_scale),
                     block_size=block_size, sel=_addr(sel), sel_count=_addr(sel_count),
                     max_sel=sel.shape[2], window=int(window), o=_addr(o), lse=_addr(lse))


def _byref_or_null(x, ctype):
    return ctypes.byref(x) if x is not None else ctypes.POINTER(ctype)()


def fused_workspace_size(verify=None, draft=None, chained=False) -> int:
    n = _lib.sss_fused_workspace_size(_byref_or_null(verify, VerifyStep),
                                      _byref_or_null(draft, DraftStep), int(bool(chained)))
    if n == 0 and _lib.sss_last_error():
        raise SSSError(SSS_ERR_INVALID_ARGUMENT, "sss_fused_workspace_size")
    return n


FUSED_FORMS = {0: "nothing", 1: "persistent", 2: "two_launch", 3: "work_list",
               4: "rows_split"}


def fused_step_form(verify=None, draft=None, chained=False) -> str:
    """sss_fused_step_form: the launch form sss_fused_step takes for these
    arguments ('persistent', 'two_launch', 'work_list' or 'nothing')."""
    f = _lib.sss_fused_step_form(_byref_or_null(verify, VerifyStep),
                                 _byref_or_null(draft, DraftStep), 1 if chained else 0)
    if f < 0:
        raise SSSError(SSS_ERR_INVALID_ARGUMENT, "sss_fused_step_form")
    return FUSED_FORMS[f]


def fused_step(verify=None, draft=None, chained=False, ws=None, device=None, verify_done=None):
    """sss_fused_step: the verify half and the draft half of a step (chained:
    the draft half drafts the verify requests over the selection this call
    makes).  verify_done: a hipEvent_t handle (int or ctypes.c_void_p) that
    sss_fused_step_marked records after the launch producing the verify
    outputs."""
    if ws is None:
        ws = workspace(fused_workspace_size(verify, draft, chained), device or "cuda")
    if verify_done is None:
        _check(_lib.sss_fused_step(_byref_or_null(verify, VerifyStep),
                                   _byref_or_null(draft, DraftStep), int(bool(chained)), _ptr(ws),
                                   ws.numel(), _stream()),
               "sss_fused_step")
    else:
        _check(_lib.sss_fused_step_marked(_byref_or_null(verify, VerifyStep),
                                          _byref_or_null(draft, DraftStep), int(bool(chained)),
                                          _ptr(ws), ws.numel(), _stream(), verify_done),
               "sss_fused_step_marked")


def kv_write(kv: PagedKV, k_new, v_new, pos0):
    """sss_kv_write: rows k_new / v_new [B][n_new][Hkv][d] to positions
    pos0[b] + i of the paged cache kv describes (the cache is written)."""
    B, n_new = k_new.shape[0], k_new.shape[1]
    _requests(kv, B, "kv_write")
    _expect(k_new, (B, n_new, kv.num_kv_heads, kv.head_dim), "k_new", _TORCH_DTYPE.get(kv.dtype))
    _expect(v_new, k_new.shape, "v_new", k_new.dtype)
    _expect(pos0, (B,), "pos0", torch.int32)
    _check(_lib.sss_kv_write(ctypes.byref(kv), _ptr(k_new), _ptr(v_new), B, n_new, _ptr(pos0),
                             _stream()),
           "sss_kv_write")


def kv_commit(seq_lens, keep, n_q, out=None):
    """sss_kv_commit: lengths after keeping keep[b] of the last n_q positions
    (in place when out is None)."""
    out = seq_lens if out is None else out
    _expect(seq_lens, (seq_lens.shape[0],), "seq_lens", torch.int32)
    _expect(keep, seq_lens.shape, "keep", torch.int32)
    _expect(out, seq_lens.shape, "out", torch.int32)
    _check(_lib.sss_kv_commit(_ptr(seq_lens), _ptr(keep), seq_lens.shape[0], int(n_q), _ptr(out),
                              _stream()),
           "sss_kv_commit")
    return out


def raw():
    """The ctypes library handle (tests call entry points with raw values)."""
    return _lib
