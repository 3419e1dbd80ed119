#!/usr/bin/env python3
"""Benchmark of the sparse self-speculative decode attention hot path on one
MI355X.

One step = one pass of the whole path over one batch:
  sss_verify_attn (k+1 queries per request over the full paged KV, block
  scores) -> sss_block_topk (critical-block lists) -> sss_draft_attn (one
  query per request over the selected blocks plus the recent window).
Default workload: batch 128, 8192-token contexts, Qwen3-8B attention shape
(32 query heads, 8 KV heads, head dim 128), k = 4, 16-token blocks and pages,
5% block budget plus a 64-token window, bf16 -- the batch-128 x 8K decode
configuration on which the bandwidth target is stated.  Inputs are seeded
synthetic tensors, resident in HBM before timing starts.

Prints one JSON line (metric, value = query tokens/s, roofline of the verify
kernel, CPU-oracle baseline on a bounded sample).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verify+draft attn tokens/s and KV HBM GB/s (% of MI355X peak), 1 GPU"
HBM_PEAK_GBS = 8000.0

# hipEventCreateWithFlags flag: the record skips the system-scope release
# fence (an L2 writeback and invalidate) that a default HIP event performs.
# These events only time work on the stream; their times are read after a
# device synchronisation, which fences by itself.
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class TimingEvent:
    """A HIP timing event without the system fence, recorded on torch's
    current stream (the stream the library launches on).  Used like a
    timing torch.cuda.Event: record(), then elapsed_time(end) in ms once
    both are complete."""

    _hip = None

    @classmethod
    def _runtime(cls):
        if cls._hip is None:
            import ctypes
            # the HIP runtime torch already loaded (one runtime per process)
            with open("/proc/self/maps") as f:
                paths = {ln.split()[-1] for ln in f if "libamdhip64.so" in ln}
            if len(paths) != 1:
                raise RuntimeError(f"expected one loaded HIP runtime, found {sorted(paths)}")
            lib = ctypes.CDLL(paths.pop())
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
            lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = (ctypes, lib)
        return cls._hip

    def __init__(self):
        import torch
        torch.cuda.init()
        ct, lib = self._runtime()
        self._ct, self._lib = ct, lib
        self._ev = ct.c_void_p()
        rc = lib.hipEventCreateWithFlags(ct.byref(self._ev), HIP_EVENT_DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self):
        import torch
        rc = self._lib.hipEventRecord(self._ev, torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    @property
    def handle(self):
        """The hipEvent_t, for a library call that records it itself."""
        return self._ev

    def elapsed_time(self, end: "TimingEvent") -> float:
        ms = self._ct.c_float()
        rc = self._lib.hipEventElapsedTime(self._ct.byref(ms), self._ev, end._ev)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def __del__(self):
        # at interpreter exit the runtime may already be torn down; the
        # process end releases the event then
        if sys.is_finalizing():
            return
        if getattr(self, "_ev", None) and self._ev.value:
            self._lib.hipEventDestroy(self._ev)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_b128_l8192")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-sample", type=int, default=128,
                    help="requests the CPU oracle processes for the baseline (0 = skip)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="the CPU baseline stops taking requests after this much oracle time")
    ap.add_argument("--verify-splits", type=int, default=-1,
                    help="override num_splits of the verify call (-1: workload default)")
    ap.add_argument("--draft-splits", type=int, default=0)
    ap.add_argument("--path", choices=("auto", "separate", "fused"), default="auto",
                    help="separate: one call per stage (verify, top-N, draft); fused: "
                         "sss_fused_step (one work-list launch, plus merge launches for "
                         "split units); auto: fused for mixed batches and for few "
                         "one-row-tile units, separate otherwise (the faster of the two on "
                         "each benchmark workload)")
    ap.add_argument("--kv-update", action="store_true",
                    help="also time sss_kv_write (the k+1 speculative positions of every "
                         "request) and sss_kv_commit, outside the timed step")
    ap.add_argument("--cold-mib", type=int, default=1024,
                    help="after the timed steps, time each step again after filling a scratch "
                         "buffer of this many MiB (evicts the KV lines from L2 and the 256 MB "
                         "Infinity Cache; reported as 'cold', 0 = skip)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run device copies of this size (calibrates HBM byte counters "
                         "against a transfer of known size) and exit")
    ap.add_argument("--read-calibration-mib", type=int, default=0,
                    help="only run the library's streaming-read probe over a buffer of this "
                         "size (3 reads; the same 16-byte non-temporal loads as the attention "
                         "kernels: calibrates FETCH_SIZE against a read of known size) and exit")
    ap.add_argument("--configs", default="all",
                    help="comma-separated workloads measured after the headline, each on its "
                         "default path, into the 'configs' block of the JSON line "
                         "('all': every benchmark configuration and the two extra workloads; "
                         "'none': skip)")
    ap.add_argument("--config-cpu-seconds", type=float, default=3.0,
                    help="oracle time budget of each entry of 'configs' (0 = no CPU baseline "
                         "there)")
    ap.add_argument("--probe-mib", type=int, default=4096,
                    help="size of the streaming-read probe buffer for the 'achievable' block "
                         "(0 = skip the probes)")
    ap.add_argument("--source-hash", action="store_true",
                    help="print the hash of the library sources (stamped into profiles/) and exit")
    return ap.parse_args()


COUNTERS = os.path.join(ROOT, "profiles", "verify_decode_b128_l8192_counters.json")
# every source the library is built from: a profile or counter summary taken
# on another build is not quoted
SOURCE_DIRS = ["sparse_self_speculative_sss_amd/csrc", "include"]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for d in SOURCE_DIRS:
        for name in sorted(os.listdir(os.path.join(ROOT, d))):
            if name.endswith((".hip", ".h")):
                h.update(f"{d}/{name}\n".encode())
                with open(os.path.join(ROOT, d, name), "rb") as f:
                    h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per verify launch from the committed counter summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by a copy of known size), or None
    when the kernel sources changed since the counters were taken."""
    try:
        with open(COUNTERS) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("workload") != workload or rec.get("source_sha256") != kernel_source_hash():
        return None
    return int(rec["hbm_bytes_per_launch"])


def algorithmic_bytes(wl, sel_np, cnt_np):
    """Bytes the method must move per step: K and V of every attended token
    read once, plus queries, outputs, LSEs, scores, selections, page tables."""
    s = wl.shape
    vb, db = wl.verify, wl.draft
    el = 2 if s.dtype == "bf16" else 4
    verify = kv_verify = topk = 0
    if vb is not None:
        lens = vb.seq_lens.cpu().numpy()
        kv_verify = int(sum(int(L) for L in lens)) * s.Hkv * s.d * el * 2
        B, n_q = vb.B, s.n_q
        q_bytes = B * n_q * s.Hq * s.d * el
        verify = (kv_verify + 2 * q_bytes + B * n_q * s.Hq * 4 + B * s.Hkv * wl.max_blocks * 4
                  + sum(-(-int(L) // s.page_size) for L in lens) * 4 + B * 4)
        topk = (B * s.Hkv * wl.max_blocks * 4 + B * s.Hkv * wl.max_sel * 4 + B * s.Hkv * 4
                + 2 * B * 4)
    toks = draft = 0
    if db is not None:
        dl = db.seq_lens.cpu().numpy()
        for b in range(db.B):
            L = int(dl[b])
            ws = L if s.window <= 0 else max(0, L - s.window)
            for h in range(s.Hkv):
                n = 0
                for j in sel_np[b, h, :cnt_np[b, h]]:
                    n += max(0, min((int(j) + 1) * s.block_size, ws) - int(j) * s.block_size)
                toks += n + (L - ws)
        draft = (toks * s.d * el * 2 + 2 * db.B * s.Hq * s.d * el + db.B * s.Hq * 4
                 + db.B * s.Hkv * (wl.max_sel + 1) * 4
                 + sum(-(-int(L) // s.page_size) for L in dl) * 4)
    return {"verify": verify, "verify_kv": kv_verify, "topk": topk, "draft": draft,
            "draft_kv": toks * s.d * el * 2, "total": verify + topk + draft}


def _request_copy(wl, batch, b):
    """Host fp64 copy of request b's pages (all KV heads), page table remapped."""
    import numpy as np
    from sparse_self_speculative_sss_amd import workload as W
    P = wl.shape.page_size
    L = int(batch.seq_lens[b])
    n = -(-L // P)
    pages = batch.page_table[b, :n].long().to(wl.k_cache.device)
    k = W.to_numpy64(wl.k_cache[pages])
    v = W.to_numpy64(wl.v_cache[pages])
    return k, v, np.arange(n, dtype=np.int32)[None], np.array([L], dtype=np.int32)


def cpu_baseline(wl, n_req, budget_s=20.0):
    """Time the fp64 oracle (as it stands) on up to n_req verify requests
    (verify + block scores + Top-N) and up to n_req draft requests (draft over
    the selection: the oracle's own for verify->draft workloads, the given
    lists for the mixed batch), taking no further request once budget_s
    seconds of oracle time are spent.  Returns query tokens/s."""
    import numpy as np
    import oracle
    from sparse_self_speculative_sss_amd import workload as W
    s = wl.shape
    vb, db = wl.verify, wl.draft
    shared = s.p_verify is None
    elapsed, tokens, nv, nd = 0.0, 0, 0, 0
    if vb is not None:
        nv = min(n_req, vb.B)
        q = W.to_numpy64(vb.q[:nv])
        qd = W.to_numpy64(db.q[:nv]) if shared else None
        done = 0
        for b in range(nv):
            if elapsed >= budget_s:
                break
            done += 1
            k, v, table, lens = _request_copy(wl, vb, b)
            t0 = time.perf_counter()
            _, _, sc = oracle.verify_with_scores(q[b:b + 1], k, v, table, lens, wl.sm_scale,
                                                 s.block_size, wl.max_blocks)
            sel, cnt = oracle.block_topk(sc.astype(np.float32), lens, s.block_size,
                                         vb.budget[b:b + 1].cpu().numpy(), s.window, wl.max_sel)
            if shared:
                oracle.draft(qd[b:b + 1], k, v, table, lens, sel, cnt, s.block_size, s.window,
                             wl.sm_scale)
            elapsed += time.perf_counter() - t0
            tokens += s.n_q + (1 if shared else 0)
            del k, v
        nv = done
    if not shared and db is not None:
        nd = min(n_req, db.B)
        qd = W.to_numpy64(db.q[:nd])
        sel_all, cnt_all = db.sel.cpu().numpy(), db.sel_count.cpu().numpy()
        done = 0
        for b in range(nd):
            if elapsed >= 2 * budget_s:
                break
            done += 1
            k, v, table, lens = _request_copy(wl, db, b)
            t0 = time.perf_counter()
            oracle.draft(qd[b:b + 1], k, v, table, lens, sel_all[b:b + 1], cnt_all[b:b + 1],
                         s.block_size, s.window, wl.sm_scale)
            elapsed += time.perf_counter() - t0
            tokens += 1
            del k, v
        nd = done
    what = (f"{nv} of {vb.B if vb else 0} verify requests" +
            ("" if shared else f" and {nd} of {db.B if db else 0} draft requests"))
    return {"value": tokens / elapsed, "unit": "tokens/s", "cores": host_cores(),
            "blas_threads": blas_threads(), "kind": "oracle",
            "sample": (f"{what} (all {s.Hkv} KV heads each): fp64 verify + block scores, Top-N "
                       f"and draft, {elapsed:.1f} s wall on the host")}


def host_cores():
    """Host cores this process may run on (the oracle's NumPy/BLAS calls use
    them; its Python loops use one)."""
    return len(os.sched_getaffinity(0))


def blas_threads():
    from threadpoolctl import threadpool_info
    return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])


def sparse_bytes(wl):
    """Sparse verification: K and V of the union of each unit's layouts (plus
    the window) read once, queries, outputs, LSEs, layouts, page tables; and,
    for comparison, the KV bytes if every query position loaded its own
    blocks separately."""
    s = wl.shape
    vb = wl.verify
    el = 2 if s.dtype == "bf16" else 4
    lens = vb.seq_lens.cpu().numpy()
    rs, rc = vb.row_sel.cpu().numpy(), vb.row_sel_count.cpu().numpy()
    union_toks = per_pos_toks = 0
    for b in range(vb.B):
        L = int(lens[b])
        ws = L if s.window <= 0 else max(0, L - s.window)
        ncand = -(-ws // s.block_size)
        for h in range(s.Hkv):
            blocks = set()
            for i in range(s.n_q):
                c = max(0, min(int(rc[b, h, i]), rs.shape[3]))
                mine = {int(j) for j in rs[b, h, i, :c] if 0 <= int(j) < ncand}
                blocks |= mine
                per_pos_toks += sum(min((j + 1) * s.block_size, ws) - j * s.block_size
                                    for j in mine) + (L - ws)
            union_toks += sum(min((j + 1) * s.block_size, ws) - j * s.block_size
                              for j in blocks) + (L - ws)
    kv = union_toks * s.d * el * 2
    q_bytes = vb.B * s.n_q * s.Hq * s.d * el
    total = (kv + 2 * q_bytes + vb.B * s.n_q * s.Hq * 4 + rs.size * 4 + rc.size * 4
             + sum(-(-int(L) // s.page_size) for L in lens) * 4 + vb.B * 4)
    return {"total": total, "kv": kv, "kv_per_position": per_pos_toks * s.d * el * 2}


def run_sparse(args, wl, dev, compact=False, cpu_seconds=None):
    """One step = one sss_sparse_verify_attn call over the batch (every
    position attends to its own layout; each unit's union is loaded once).
    Prints the JSON line, or with compact=True returns a 'configs' entry."""
    import numpy as np
    import torch
    import oracle
    from sparse_self_speculative_sss_amd import sss
    from sparse_self_speculative_sss_amd import workload as W
    s = wl.shape
    vb = wl.verify
    B, n_q = vb.B, s.n_q
    kv = sss.paged_kv(wl.k_cache, wl.v_cache, vb.page_table, vb.seq_lens, vb.max_seq_len)
    o = torch.empty_like(vb.q)
    lse = torch.empty((B, n_q, s.Hq), dtype=torch.float32, device=dev)
    splits = max(0, args.verify_splits)
    ws = sss.workspace(sss.sparse_verify_workspace_size(kv, B, n_q, s.Hq, s.block_size,
                                                        vb.row_sel.shape[3], s.window, splits),
                       dev)

    def step():
        sss.sparse_verify_attn(kv, vb.q, wl.sm_scale, s.block_size, vb.row_sel,
                               vb.row_sel_count, s.window, o, lse, ws=ws, num_splits=splits)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    nb = sparse_bytes(wl)
    evs = [[TimingEvent() for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs[i][0].record()
        step()
        evs[i][1].record()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    k_list = [e[0].elapsed_time(e[1]) for e in evs]
    k_ms = float(np.mean(k_list))
    gbs = nb["total"] / (k_ms * 1e-3) / 1e9

    # the same loads without grouping: one launch per query position, each
    # holding only that position's layout (every KV block a position selects
    # is loaded once per position; outputs go to scratch and are not used)
    solo = []
    for i in range(n_q):
        rc_i = torch.zeros_like(vb.row_sel_count)
        rc_i[:, :, i] = vb.row_sel_count[:, :, i]
        solo.append(rc_i)
    o_s, lse_s = torch.empty_like(o), torch.empty_like(lse)

    def ungrouped():
        for rc_i in solo:
            sss.sparse_verify_attn(kv, vb.q, wl.sm_scale, s.block_size, vb.row_sel, rc_i,
                                   s.window, o_s, lse_s, ws=ws, num_splits=splits)

    for _ in range(2):
        ungrouped()
    eu = [TimingEvent() for _ in range(2)]
    eu[0].record()
    for _ in range(args.steps):
        ungrouped()
    eu[1].record()
    torch.cuda.synchronize()
    u_ms = eu[0].elapsed_time(eu[1]) / args.steps
    rec = {
        "metric": "sparse verify attn tokens/s and KV HBM GB/s (% of MI355X peak), 1 GPU",
        "value": round(B * n_q / (ms_step / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": s.dtype,
        "data": "synthetic (seeded; Qwen3-8B attention shape, per-position layouts sharing "
                f"{int(round(100 * s.layout_shared))}% of their blocks)",
        "config": {"workload": s.name, "batch": B, "context": int(vb.seq_lens.max()),
                   "q_heads": s.Hq, "kv_heads": s.Hkv, "head_dim": s.d, "k_plus_1": n_q,
                   "block": s.block_size, "page": s.page_size, "window": s.window,
                   "layout_blocks": int(vb.row_sel_count.max()),
                   "layout_shared": s.layout_shared, "splits": splits},
        "roofline": {
            "kernel": "sss_sparse_verify_attn (attn_mfma_kernel<sparse verify>; split merge "
                      "launch included when units are split)",
            "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
            "algorithmic_bytes": nb["total"], "ms": round(k_ms, 4),
        },
        "grouping": {"kv_bytes_union": nb["kv"], "kv_bytes_per_position": nb["kv_per_position"],
                     "ratio": round(nb["kv_per_position"] / max(1, nb["kv"]), 3),
                     "grouped_ms": round(k_ms, 4),
                     "one_launch_per_position_ms": round(u_ms, 4),
                     "speedup": round(u_ms / k_ms, 3)},
    }
    budget = args.cpu_seconds if cpu_seconds is None else cpu_seconds
    if args.cpu_sample > 0 and budget > 0:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        n = min(args.cpu_sample, B)
        q = W.to_numpy64(vb.q[:n])
        rs, rc = vb.row_sel.cpu().numpy(), vb.row_sel_count.cpu().numpy()
        elapsed = 0.0
        done = 0
        for b in range(n):
            if elapsed >= budget:
                break
            done += 1
            k, v, table, lens = _request_copy(wl, vb, b)
            t0 = time.perf_counter()
            oracle.sparse_verify(q[b:b + 1], k, v, table, lens, rs[b:b + 1], rc[b:b + 1],
                                 s.block_size, s.window, wl.sm_scale)
            elapsed += time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": done * n_q / elapsed, "unit": "tokens/s",
                               "cores": host_cores(), "blas_threads": blas_threads(),
                               "kind": "oracle",
                               "sample": f"{done} of {B} requests (all {s.Hkv} KV heads each): fp64 "
                                         f"sparse verify, {elapsed:.1f} s wall on the host"}
    else:
        rec["cpu_baseline"] = None
    if compact:
        med = float(np.median(k_list))
        return {"workload": s.name, "path": "sparse_verify", "dtype": s.dtype,
                "verify_requests": B, "draft_requests": 0, "query_tokens_per_step": B * n_q,
                "ms_per_step_wall": round(ms_step, 4), "ms_per_step_median": round(med, 4),
                "ms_per_step_p10": pct(k_list, 10), "ms_per_step_p90": pct(k_list, 90),
                "tokens/s": round(B * n_q / (med * 1e-3), 1), "algorithmic_bytes": nb["total"],
                "GB/s": round(nb["total"] / (med * 1e-3) / 1e9, 1),
                "frac": round(nb["total"] / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "kv_bytes": nb["kv"], "dominant": rec["roofline"], "grouping": rec["grouping"],
                "cpu_baseline": rec["cpu_baseline"]}
    print(json.dumps(rec), flush=True)


def time_kv_update(wl, kv, vb, dev, steps):
    """sss_kv_write of the last n_q positions of every verify request (the
    values already there, so the cache is unchanged) and sss_kv_commit keeping
    all of them (lengths unchanged); mean times over `steps` calls each."""
    import torch
    from sparse_self_speculative_sss_amd import sss
    s = wl.shape
    B, n_q = vb.B, s.n_q
    lens = vb.seq_lens
    pos0 = (lens - n_q).to(torch.int32)
    # the rows currently stored at those positions
    P = s.page_size
    t = pos0[:, None].long() + torch.arange(n_q, device=dev)[None]
    pages = torch.gather(vb.page_table.long(), 1, t // P)
    k_new = wl.k_cache[pages, :, t % P].contiguous()        # [B][n_q][Hkv][d]
    v_new = wl.v_cache[pages, :, t % P].contiguous()
    keep = torch.full((B,), n_q, dtype=torch.int32, device=dev)
    out = torch.empty_like(lens)
    ev = [TimingEvent() for _ in range(3)]
    for _ in range(3):
        sss.kv_write(kv, k_new, v_new, pos0)
        sss.kv_commit(lens, keep, n_q, out)
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(steps):
        sss.kv_write(kv, k_new, v_new, pos0)
    ev[1].record()
    for _ in range(steps):
        sss.kv_commit(lens, keep, n_q, out)
    ev[2].record()
    torch.cuda.synchronize()
    w_ms = ev[0].elapsed_time(ev[1]) / steps
    c_ms = ev[1].elapsed_time(ev[2]) / steps
    moved = 2 * k_new.numel() * k_new.element_size() * 2      # K and V, read + written
    return {"write_ms": round(w_ms, 4), "write_bytes": moved,
            "write_GB/s": round(moved / (w_ms * 1e-3) / 1e9, 1), "commit_ms": round(c_ms, 4)}


def default_path(s):
    """The faster path on MI355X for a workload: the fused step for mixed
    batches and for chained steps of one-row-tile units on the matrix-core
    path (16 requests x 4K: 0.076 against 0.096 ms; batch 128 x 8K, where
    one wave per unit selects and drafts after the verify launch: 0.723
    against 0.728 ms); the per-stage calls with several row tiles per unit,
    or on the vector-ALU and single-token paths, which the fused step does
    not take.  (On the 80-row long context the fused step takes its
    rows-split form, the per-stage kernels without the Top-N launch:
    0.145-0.146 against 0.144-0.145 ms for the per-stage calls.)"""
    shared = s.p_verify is None
    one_tile = s.n_q * (s.Hq // s.Hkv) <= 32
    mfma = s.dtype == "bf16" and s.block_size % 16 == 0 and s.page_size % 16 == 0
    return "fused" if (not shared or (one_tile and mfma)) else "separate"


def pct(x, q):
    import numpy as np
    return round(float(np.percentile(np.asarray(x), q)), 4)


def run_step_workload(args, wl, dev, path="auto", steps=20, warmup=5, cold_mib=0,
                      verify_splits=-1, draft_splits=0):
    """Warm-up, then `steps` timed steps of the whole path (verify, Top-N,
    draft) with events at every step boundary and after each verify call,
    then (untimed) a stage breakdown and, with cold_mib, each step again
    after a scratch fill that evicts the caches.  Returns the raw results."""
    import numpy as np
    import torch
    from sparse_self_speculative_sss_amd import sss
    s = wl.shape
    vb, db = wl.verify, wl.draft
    shared = s.p_verify is None      # draft reads the selection this step's verify made
    if path == "auto":
        path = default_path(s)
    n_q = s.n_q
    Bv = vb.B if vb is not None else 0
    Bd = db.B if db is not None else 0
    vsplits = s.num_splits if verify_splits < 0 else verify_splits
    verify_launches = 0
    if Bv:
        kv_v = sss.paged_kv(wl.k_cache, wl.v_cache, vb.page_table, vb.seq_lens, vb.max_seq_len)
        o = torch.empty_like(vb.q)
        lse = torch.empty((Bv, n_q, s.Hq), dtype=torch.float32, device=dev)
        sc = torch.empty((Bv, s.Hkv, wl.max_blocks), dtype=torch.float32, device=dev)
        sel = torch.empty((Bv, s.Hkv, wl.max_sel), dtype=torch.int32, device=dev)
        cnt = torch.empty((Bv, s.Hkv), dtype=torch.int32, device=dev)
        nws = sss.verify_workspace_size(kv_v, Bv, n_q, s.Hq, s.block_size, wl.max_blocks, vsplits)
        ws_v = sss.workspace(nws, dev)
        # one launch when the plan keeps every unit in one chunk: the same
        # workspace as an explicit single split (a split plan adds partials)
        one = sss.verify_workspace_size(kv_v, Bv, n_q, s.Hq, s.block_size, wl.max_blocks, 1)
        verify_launches = 1 if (nws == one and s.dtype == "bf16") else 2
    if Bd:
        kv_d = sss.paged_kv(wl.k_cache, wl.v_cache, db.page_table, db.seq_lens, db.max_seq_len)
        od = torch.empty_like(db.q)
        lsed = torch.empty((Bd, 1, s.Hq), dtype=torch.float32, device=dev)
        sel_d = sel if shared else db.sel
        cnt_d = cnt if shared else db.sel_count
        ws_d = sss.workspace(sss.draft_workspace_size(kv_d, Bd, s.Hq, s.block_size, wl.max_sel,
                                                      s.window, draft_splits), dev)
    if path == "fused":
        v_step = d_step = None
        if Bv:
            v_step = sss.verify_step(kv_v, vb.q, wl.sm_scale, s.block_size, wl.max_blocks, o, lse,
                                     sc, budget=vb.budget, window=s.window, sel=sel,
                                     sel_count=cnt)
        if Bd:
            # a shared workload drafts the verify requests over this step's
            # selection (same cache description); a mixed one its own
            d_step = sss.draft_step(kv_v if shared else kv_d, db.q, wl.sm_scale, s.block_size,
                                    sel_d, cnt_d, s.window, od, lsed)
        ws_f = sss.workspace(sss.fused_workspace_size(v_step, d_step, shared), dev)
        form = sss.fused_step_form(v_step, d_step, shared)

    # mark: event at the start of the step; mid: after the verify call (the
    # roofline kernel); top / end: after Top-N and the draft (stage pass only)
    def step(mark=None, mid=None, top=None, end=None):
        if mark is not None:
            mark.record()
        if path == "fused":
            sss.fused_step(v_step, d_step, chained=shared, ws=ws_f,
                           verify_done=None if mid is None else mid.handle)
            return
        if Bv:
            sss.verify_attn(kv_v, vb.q, wl.sm_scale, s.block_size, wl.max_blocks, o, lse, sc,
                            ws=ws_v, num_splits=vsplits)
        if mid is not None:
            mid.record()
        if Bv:
            sss.block_topk(sc, vb.seq_lens, s.block_size, vb.budget, s.window, sel, cnt)
        if top is not None:
            top.record()
        if Bd:
            sss.draft_attn(kv_d, db.q, wl.sm_scale, s.block_size, sel_d, cnt_d, s.window, od,
                           lsed, ws=ws_d, num_splits=draft_splits)
        if end is not None:
            end.record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    nbytes = algorithmic_bytes(wl, sel_d.cpu().numpy() if Bd else None,
                               cnt_d.cpu().numpy() if Bd else None)

    # timed steps: consecutive steps share their boundary event (one record
    # per step boundary, plus one after each verify call on the per-stage
    # path, or after the verify launch inside the fused step's two-launch
    # form); every record is a barrier on the stream
    marks = [TimingEvent() for _ in range(steps + 1)]
    timed_mid = path == "separate" or (path == "fused" and form in ("two_launch", "rows_split"))
    mids = [TimingEvent() for _ in range(steps)] if timed_mid else None
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(marks[i], mids[i] if mids else None)
    marks[-1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_ms = [marks[i].elapsed_time(marks[i + 1]) for i in range(steps)]
    verify_ms = ([marks[i].elapsed_time(mids[i]) for i in range(steps)] if mids else
                 list(step_ms))
    # stage breakdown (untimed pass; the fused two-launch form's selection
    # and draft launch is the rest of each timed step)
    t_ms = d_ms = sd_ms = None
    if path == "fused" and mids:
        sd_ms = float(np.mean([a - b for a, b in zip(step_ms, verify_ms)]))
    if path == "separate":
        sev = [[TimingEvent() for _ in range(4)] for _ in range(steps)]
        for i in range(steps):
            step(*sev[i])
        torch.cuda.synchronize()
        t_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in sev]))
        d_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in sev]))
    cold = None
    if cold_mib > 0:
        scratch = torch.empty(cold_mib << 20, dtype=torch.uint8, device=dev)
        cev = [[TimingEvent() for _ in range(2)] for _ in range(steps)]
        for i in range(steps):
            scratch.fill_(i & 255)
            cev[i][0].record()
            step()
            cev[i][1].record()
        torch.cuda.synchronize()
        cold = [e[0].elapsed_time(e[1]) for e in cev]
        del scratch
    res = dict(path=path, form=form if path == "fused" else None, Bv=Bv, Bd=Bd, n_q=n_q,
               vsplits=vsplits, draft_splits=draft_splits,
               verify_launches=verify_launches, steps=steps, warmup=warmup,
               ms_wall=(t1 - t0) * 1e3 / steps, step_ms=step_ms, verify_ms=verify_ms,
               topk_ms=t_ms, draft_ms=d_ms, select_draft_ms=sd_ms, cold=cold,
               cold_mib=cold_mib, nbytes=nbytes,
               tokens=Bv * n_q + Bd)
    if Bv:
        res["kv_v"] = kv_v
    return res


def roofline_of(res, workload):
    """Roofline block of the dominant kernel: the verify call (one launch of
    attn_mfma_kernel when units run unsplit), or the whole fused call."""
    import numpy as np
    nb = res["nbytes"]
    v_ms = float(np.mean(res["verify_ms"]))
    if res["path"] == "fused" and res.get("form") == "two_launch":
        # the verify launch inside the step, timed by the event the step
        # records after it (the same kernel as the per-stage verify call)
        a = nb["verify"] / (v_ms * 1e-3) / 1e9
        return {"kernel": "attn_mfma_kernel<verify> (the first launch of sss_fused_step's "
                          "two-launch form: every unit in one chunk)",
                "bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(a / HBM_PEAK_GBS, 4), "traffic": measured_traffic(workload),
                "algorithmic_bytes": nb["verify"], "ms": round(v_ms, 4)}
    if res["path"] == "fused" and res.get("form") == "rows_split":
        # the verify and merge launches inside the step, timed by the event
        # the step records after the merge
        a = nb["verify"] / (v_ms * 1e-3) / 1e9
        return {"kernel": "verify_rows_kernel + finalize_kernel (the verify and merge launches "
                          "of sss_fused_step's rows-split form)",
                "bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(a / HBM_PEAK_GBS, 4), "traffic": None,
                "algorithmic_bytes": nb["verify"], "ms": round(v_ms, 4)}
    if res["path"] == "fused":
        a = nb["total"] / (v_ms * 1e-3) / 1e9
        kernels = {
            "persistent": "sss_fused_step (one persistent launch: verify, scores, Top-N and "
                          "draft of every unit)",
        }
        return {"kernel": kernels.get(res.get("form"),
                                      "sss_fused_step (its work-list launch plus the merge, "
                                      "selection and draft launches of split units)"),
                "bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(a / HBM_PEAK_GBS, 4), "traffic": None,
                "algorithmic_bytes": nb["total"], "ms": round(v_ms, 4)}
    a = nb["verify"] / (v_ms * 1e-3) / 1e9 if res["Bv"] else 0.0
    one = res["verify_launches"] == 1
    return {"kernel": ("attn_mfma_kernel<verify> (the one launch of sss_verify_attn: every "
                       "unit in one chunk)" if one else
                       "sss_verify_attn (attention launch plus the split merge / scoring launch)"),
            "bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(a / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(workload) if one else None,
            "algorithmic_bytes": nb["verify"], "ms": round(v_ms, 4)}


def config_record(res, wl, cpu=None):
    """Compact per-workload record for the 'configs' block."""
    import numpy as np
    s = wl.shape
    nb = res["nbytes"]
    med = float(np.median(res["step_ms"]))
    kv = nb["verify_kv"] + nb["draft_kv"]
    rec = {
        "workload": s.name, "path": res["path"], "dtype": s.dtype,
        **({"form": res["form"]} if res.get("form") else {}),
        "verify_requests": res["Bv"], "draft_requests": res["Bd"],
        "query_tokens_per_step": res["tokens"],
        "ms_per_step_wall": round(res["ms_wall"], 4),
        "ms_per_step_median": round(med, 4),
        "ms_per_step_p10": pct(res["step_ms"], 10), "ms_per_step_p90": pct(res["step_ms"], 90),
        "tokens/s": round(res["tokens"] / (med * 1e-3), 1),
        "algorithmic_bytes": nb["total"],
        "GB/s": round(nb["total"] / (med * 1e-3) / 1e9, 1),
        "frac": round(nb["total"] / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "kv_bytes": kv,
        "kv_frac": round(kv / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "dominant": roofline_of(res, s.name),
    }
    if res["topk_ms"] is not None:
        rec["topk_ms"] = round(res["topk_ms"], 4)
        rec["draft_ms"] = round(res["draft_ms"], 4)
    if res["cold"]:
        c = float(np.median(res["cold"]))
        rec["cold_ms_median"] = round(c, 4)
        rec["cold_frac"] = round(nb["total"] / (c * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    if cpu is not None:
        rec["cpu_baseline"] = cpu
    return rec


def probes(dev, kv, batch, mib, reps=5):
    """Achievable read rates from the library's probe kernels: a plain
    streaming read of `mib` MiB, and a read of exactly the (page, head) runs
    the verify loads (the same bytes in the permuted page order)."""
    import ctypes
    import numpy as np
    import torch
    from sparse_self_speculative_sss_amd import sss
    lib = sss.raw()
    lib.sss_probe_stream_read.restype = ctypes.c_int32
    lib.sss_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                          ctypes.c_void_p]
    lib.sss_probe_paged_read.restype = ctypes.c_int32
    lib.sss_probe_paged_read.argtypes = [ctypes.POINTER(sss.PagedKV), ctypes.c_int32,
                                         ctypes.c_void_p, ctypes.c_void_p]
    sink = torch.zeros(4096, dtype=torch.int32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    buf = torch.ones(mib << 20, dtype=torch.uint8, device=dev)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ev = [TimingEvent() for _ in range(reps + 1)]
        for i in range(reps):
            ev[i].record()
            fn()
        ev[-1].record()
        torch.cuda.synchronize()
        return [ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]

    def stream_read():
        st = lib.sss_probe_stream_read(buf.data_ptr(), buf.numel(), sink.data_ptr(), stream)
        if st != 0:
            raise RuntimeError(f"sss_probe_stream_read failed ({st})")

    def paged_read():
        st = lib.sss_probe_paged_read(ctypes.byref(kv), batch, sink.data_ptr(), stream)
        if st != 0:
            raise RuntimeError(f"sss_probe_paged_read failed ({st})")

    ts = timed(stream_read)
    del buf
    tp = timed(paged_read)
    return ts, tp


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(attention units shard by request and KV head with no exchange; only the one-GPU share is measured)",
              file=sys.stderr)
        sys.exit(2)
    if args.source_hash:
        print(kernel_source_hash())
        return

    import numpy as np
    import torch
    from sparse_self_speculative_sss_amd import workload as W
    from sparse_self_speculative_sss_amd import sss

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": {"bytes_read": n * 4, "bytes_written": n * 4,
                                               "copies": 3}}), flush=True)
        return
    if args.read_calibration_mib > 0:
        import ctypes
        lib = sss.raw()
        lib.sss_probe_stream_read.restype = ctypes.c_int32
        lib.sss_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                              ctypes.c_void_p]
        n = args.read_calibration_mib << 20
        buf = torch.ones(n, dtype=torch.uint8, device=dev)
        sink = torch.zeros(4096, dtype=torch.int32, device=dev)
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for _ in range(3):
            if lib.sss_probe_stream_read(buf.data_ptr(), n, sink.data_ptr(), stream) != 0:
                raise RuntimeError("sss_probe_stream_read failed")
        torch.cuda.synchronize()
        print(json.dumps({"read_calibration": {"bytes_read": n, "reads": 3,
                                               "kernel": "sss::stream_read_kernel"}}), flush=True)
        return
    print(f"[bench] generating {args.workload} seed={args.seed}", file=sys.stderr, flush=True)
    wl = W.make(args.workload, seed=args.seed, device=dev)
    s = wl.shape
    if s.layout_shared is not None:
        run_sparse(args, wl, dev)
        return
    res = run_step_workload(args, wl, dev, path=args.path, steps=args.steps, warmup=args.warmup,
                            cold_mib=args.cold_mib, verify_splits=args.verify_splits,
                            draft_splits=args.draft_splits)
    vb, db = wl.verify, wl.draft
    Bv, Bd, n_q = res["Bv"], res["Bd"], res["n_q"]
    nbytes = res["nbytes"]
    ms_step = res["ms_wall"]
    step_ms = res["step_ms"]
    v_ms = float(np.mean(res["verify_ms"]))
    value = res["tokens"] / (ms_step / 1e3)
    unit_gbs = nbytes["total"] / (ms_step * 1e-3) / 1e9
    roofline = roofline_of(res, s.name)
    lens = vb.seq_lens if Bv else db.seq_lens
    med = float(np.median(step_ms))
    rec = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": s.dtype,
        "data": "synthetic (seeded; Qwen3-8B attention shape, planted heavy-hitter keys)",
        "config": {
            "workload": s.name, "batch": s.B, "verify_requests": Bv, "draft_requests": Bd,
            "context": (int(lens.max()) if s.p_verify is None
                        else f"{int(lens.min())}..{int(lens.max())}"),
            "q_heads": s.Hq, "kv_heads": s.Hkv, "head_dim": s.d, "k_plus_1": n_q,
            "block": s.block_size, "page": s.page_size, "window": s.window,
            "budget_blocks": (int(vb.budget[0]) if s.budget_frac is None or s.p_verify is None
                              else f"ceil({s.budget_frac} * blocks)"),
            "verify_splits": res["vsplits"], "draft_splits": res["draft_splits"],
            "path": res["path"],
            **({"form": res["form"]} if res.get("form") else {}),
        },
        "roofline": roofline,
        "warm": {
            "ms_per_step_median": round(med, 4),
            "ms_per_step_p10": pct(step_ms, 10), "ms_per_step_p90": pct(step_ms, 90),
            "verify_ms_median": round(float(np.median(res["verify_ms"])), 4),
            "verify_ms_p10": pct(res["verify_ms"], 10), "verify_ms_p90": pct(res["verify_ms"], 90),
            "timing": "HIP events (no system fence) at every step boundary and after each "
                      "verify call, on the library's stream; ms_per_step is the wall-clock mean",
        },
        "step_hbm": {
            "algorithmic_bytes": nbytes["total"],
            "GB/s": round(unit_gbs, 1),
            "frac": round(unit_gbs / HBM_PEAK_GBS, 4),
            # K and V alone (every verified token once, every drafted token once)
            "kv_bytes": nbytes["verify_kv"] + nbytes["draft_kv"],
            "kv_GB/s": round((nbytes["verify_kv"] + nbytes["draft_kv"]) / (ms_step * 1e-3) / 1e9, 1),
            "kv_frac": round((nbytes["verify_kv"] + nbytes["draft_kv"]) / (ms_step * 1e-3) / 1e9
                             / HBM_PEAK_GBS, 4),
            "verify_ms": round(v_ms, 4),
            "topk_ms": None if res["topk_ms"] is None else round(res["topk_ms"], 4),
            "draft_ms": None if res["draft_ms"] is None else round(res["draft_ms"], 4),
            **({"select_draft_ms": round(res["select_draft_ms"], 4),
                "stage_times": "verify_ms from the timed steps (an event the fused step records "
                               "after its verify launch); select_draft_ms = step - verify"}
               if res.get("select_draft_ms") is not None else
               {"stage_times": "verify_ms from the timed steps; topk_ms and draft_ms from a "
                               "separate untimed pass with events between the stages"}),
            "draft_GB/s": (round(nbytes["draft"] / (res["draft_ms"] * 1e-3) / 1e9, 1)
                           if Bd and res["draft_ms"] else None),
        },
    }
    if res["cold"]:
        ct = res["cold"]
        c_med = float(np.median(ct))
        rec["cold"] = {"flush_mib": res["cold_mib"],
                       "ms_per_step_median": round(c_med, 4),
                       "ms_per_step_p10": pct(ct, 10), "ms_per_step_p90": pct(ct, 90),
                       "GB/s": round(nbytes["total"] / (c_med * 1e-3) / 1e9, 1),
                       "frac": round(nbytes["total"] / (c_med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                       "timing": "events around each step; the fill runs before the first event"}
    else:
        rec["cold"] = None
    if args.kv_update and Bv:
        rec["kv_update"] = time_kv_update(wl, res["kv_v"], vb, dev, args.steps)
    if args.probe_mib > 0 and Bv:
        print("[bench] bandwidth probes", file=sys.stderr, flush=True)
        ts, tp = probes(dev, res["kv_v"], Bv, args.probe_mib)
        sr = (args.probe_mib << 20) / (float(np.median(ts)) * 1e-3) / 1e9
        pr = nbytes["verify_kv"] / (float(np.median(tp)) * 1e-3) / 1e9
        rec["achievable"] = {
            "stream_read_GB/s": round(sr, 1), "stream_read_frac": round(sr / HBM_PEAK_GBS, 4),
            "stream_read_bytes": args.probe_mib << 20,
            "paged_read_GB/s": round(pr, 1), "paged_read_frac": round(pr / HBM_PEAK_GBS, 4),
            "paged_read_bytes": nbytes["verify_kv"],
            "verify_vs_paged_read": (round(roofline["achieved"] / pr, 4)
                                     if roofline["algorithmic_bytes"] == nbytes["verify"]
                                     else None),
            "kernels": "sss_probe_stream_read / sss_probe_paged_read (16-byte non-temporal loads, "
                       "nothing but reads): context for the roofline, not the peak",
        }
    if args.cpu_sample > 0:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(wl, args.cpu_sample, args.cpu_seconds)
    else:
        rec["cpu_baseline"] = None
    headline = config_record(res, wl, None)
    if rec["cpu_baseline"] is not None:
        headline["cpu_baseline"] = rec["cpu_baseline"]
    # a chained headline workload on the other path too (per-stage calls
    # beside the fused step, or the other way round), for comparison
    alt = None
    if args.configs != "none" and s.p_verify is None:
        other = "separate" if res["path"] == "fused" else "fused"
        print(f"[bench] config {s.name} ({other} path)", file=sys.stderr, flush=True)
        r_alt = run_step_workload(args, wl, dev, path=other, steps=args.steps,
                                  warmup=args.warmup, cold_mib=args.cold_mib)
        alt = config_record(r_alt, wl, None)
        print(f"[bench] config {s.name} ({other} path): "
              f"{alt['ms_per_step_median']} ms ({alt['frac']:.3f} of peak)",
              file=sys.stderr, flush=True)
        del r_alt
    del wl, res
    torch.cuda.empty_cache()

    names = [] if args.configs == "none" else (
        [n for n in W.SHAPE_ORDER] if args.configs == "all" else args.configs.split(","))
    configs = []
    for name in names:
        if name == s.name:
            configs.append(headline)
            if alt is not None:
                configs.append(alt)
            continue
        print(f"[bench] config {name}", file=sys.stderr, flush=True)
        w2 = W.make(name, seed=args.seed, device=dev)
        if w2.shape.layout_shared is not None:
            configs.append(run_sparse(args, w2, dev, compact=True,
                                      cpu_seconds=args.config_cpu_seconds))
            print(f"[bench] config {name}: {configs[-1]['ms_per_step_median']} ms",
                  file=sys.stderr, flush=True)
        else:
            r2 = run_step_workload(args, w2, dev, steps=args.steps, warmup=args.warmup,
                                   cold_mib=args.cold_mib)
            cpu = (cpu_baseline(w2, args.cpu_sample, args.config_cpu_seconds)
                   if args.config_cpu_seconds > 0 and args.cpu_sample > 0 else None)
            configs.append(config_record(r2, w2, cpu))
            print(f"[bench] config {name}: {configs[-1]['ms_per_step_median']} ms "
                  f"({configs[-1]['frac']:.3f} of peak)", file=sys.stderr, flush=True)
            del r2
        del w2
        torch.cuda.empty_cache()
    rec["configs"] = configs
    rec["source_sha256"] = kernel_source_hash()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
