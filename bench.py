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
    return ap.parse_args()


COUNTERS = os.path.join(ROOT, "profiles", "verify_decode_b128_l8192_counters.json")
KERNEL_SOURCES = ["sparse_self_speculative_sss_amd/csrc/attn_item.h",
                  "sparse_self_speculative_sss_amd/csrc/attn_mfma.hip",
                  "sparse_self_speculative_sss_amd/csrc/sss_common.h",
                  "sparse_self_speculative_sss_amd/csrc/api.hip"]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
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
    from threadpoolctl import threadpool_info
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
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    what = (f"{nv} of {vb.B if vb else 0} verify requests" +
            ("" if shared else f" and {nd} of {db.B if db else 0} draft requests"))
    return {"value": tokens / elapsed, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"{what} (all {s.Hkv} KV heads each): fp64 verify + block scores, Top-N "
                       f"and draft, {elapsed:.1f} s wall on the host")}


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


def run_sparse(args, wl, dev):
    """One step = one sss_sparse_verify_attn call over the batch (every
    position attends to its own layout; each unit's union is loaded once)."""
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
    k_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
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
    if args.cpu_sample > 0:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        n = min(args.cpu_sample, B)
        q = W.to_numpy64(vb.q[:n])
        rs, rc = vb.row_sel.cpu().numpy(), vb.row_sel_count.cpu().numpy()
        elapsed = 0.0
        done = 0
        for b in range(n):
            if elapsed >= args.cpu_seconds:
                break
            done += 1
            k, v, table, lens = _request_copy(wl, vb, b)
            t0 = time.perf_counter()
            oracle.sparse_verify(q[b:b + 1], k, v, table, lens, rs[b:b + 1], rc[b:b + 1],
                                 s.block_size, s.window, wl.sm_scale)
            elapsed += time.perf_counter() - t0
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        rec["cpu_baseline"] = {"value": done * n_q / elapsed, "unit": "tokens/s",
                               "cores": threads, "kind": "oracle",
                               "sample": f"{done} of {B} requests (all {s.Hkv} KV heads each): fp64 "
                                         f"sparse verify, {elapsed:.1f} s wall on the host"}
    else:
        rec["cpu_baseline"] = None
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


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(attention units shard by request and KV head with no exchange; only the one-GPU share is measured)",
              file=sys.stderr)
        sys.exit(2)

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
    print(f"[bench] generating {args.workload} seed={args.seed}", file=sys.stderr, flush=True)
    wl = W.make(args.workload, seed=args.seed, device=dev)
    s = wl.shape
    if s.layout_shared is not None:
        run_sparse(args, wl, dev)
        return
    vb, db = wl.verify, wl.draft
    shared = s.p_verify is None      # draft reads the selection this step's verify made
    if args.path == "auto":
        # the faster path on MI355X: the fused step for mixed batches and for
        # steps of few one-row-tile units on the matrix-core path (16
        # requests x 4K: 0.088 against 0.096 ms); the per-stage calls with
        # 1024 or more units (one-wave drafts; level or faster: 0.749 against
        # 0.764 ms at batch 128 x 8K), several row tiles per unit (80-row
        # long context: 0.199 against 0.201 ms), or the vector-ALU and
        # single-token paths, which the fused step does not take
        units = s.B * s.Hkv
        one_tile = s.n_q * (s.Hq // s.Hkv) <= 32
        mfma = s.dtype == "bf16" and s.block_size % 16 == 0 and s.page_size % 16 == 0
        few = units < 1024 and one_tile and mfma
        args.path = "fused" if (not shared or few) else "separate"
    n_q = s.n_q
    Bv = vb.B if vb is not None else 0
    Bd = db.B if db is not None else 0
    vsplits = s.num_splits if args.verify_splits < 0 else args.verify_splits
    if Bv:
        kv_v = sss.paged_kv(wl.k_cache, wl.v_cache, vb.page_table, vb.seq_lens, vb.max_seq_len)
        o = torch.empty_like(vb.q)
        lse = torch.empty((Bv, n_q, s.Hq), dtype=torch.float32, device=dev)
        sc = torch.empty((Bv, s.Hkv, wl.max_blocks), dtype=torch.float32, device=dev)
        sel = torch.empty((Bv, s.Hkv, wl.max_sel), dtype=torch.int32, device=dev)
        cnt = torch.empty((Bv, s.Hkv), dtype=torch.int32, device=dev)
        ws_v = sss.workspace(sss.verify_workspace_size(kv_v, Bv, n_q, s.Hq, s.block_size,
                                                       wl.max_blocks, vsplits), dev)
        # the verify call is a single kernel launch when its plan leaves units unsplit
        verify_launches = 1 if sss.verify_workspace_size(kv_v, Bv, n_q, s.Hq, s.block_size,
                                                         wl.max_blocks, vsplits) == 0 else 2
    else:
        verify_launches = 0
    if Bd:
        kv_d = sss.paged_kv(wl.k_cache, wl.v_cache, db.page_table, db.seq_lens, db.max_seq_len)
        od = torch.empty_like(db.q)
        lsed = torch.empty((Bd, 1, s.Hq), dtype=torch.float32, device=dev)
        sel_d = sel if shared else db.sel
        cnt_d = cnt if shared else db.sel_count
        ws_d = sss.workspace(sss.draft_workspace_size(kv_d, Bd, s.Hq, s.block_size, wl.max_sel,
                                                      s.window, args.draft_splits), dev)

    if args.path == "fused":
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

    # ev: events [before, after the verify (or fused) call, after Top-N,
    # after the draft]; the timed steps record only the first two (each
    # record is a barrier on the stream), a separate pass records all four
    # for the stage breakdown
    def step(ev=None, stages=False, chain=False):
        if args.path == "fused":
            if ev is not None:
                ev[0].record()
            sss.fused_step(v_step, d_step, chained=shared, ws=ws_f)
            # chain: the next step's first event (or the one after the
            # loop) closes this one
            if ev is not None and not chain:
                ev[1].record()
                if stages:
                    ev[2].record()
                    ev[3].record()
            return
        if ev is not None:
            ev[0].record()
        if Bv:
            sss.verify_attn(kv_v, vb.q, wl.sm_scale, s.block_size, wl.max_blocks, o, lse, sc,
                            ws=ws_v, num_splits=vsplits)
        if ev is not None:
            ev[1].record()
        if Bv:
            sss.block_topk(sc, vb.seq_lens, s.block_size, vb.budget, s.window, sel, cnt)
        if ev is not None and stages:
            ev[2].record()
        if Bd:
            sss.draft_attn(kv_d, db.q, wl.sm_scale, s.block_size, sel_d, cnt_d, s.window, od,
                           lsed, ws=ws_d, num_splits=args.draft_splits)
        if ev is not None and stages:
            ev[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    nbytes = algorithmic_bytes(wl, sel_d.cpu().numpy() if Bd else None,
                               cnt_d.cpu().numpy() if Bd else None)

    chain = args.path == "fused"
    if chain:
        # the fused call is the whole step: consecutive steps share their
        # boundary event, one record per step
        marks = [TimingEvent() for _ in range(args.steps + 1)]
        evs = [[marks[i], marks[i + 1]] for i in range(args.steps)]
    else:
        evs = [[TimingEvent() for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i], chain=chain)
    if chain:
        marks[-1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    v_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    # stage breakdown (untimed pass)
    sev = [[TimingEvent() for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(sev[i], stages=True)
    torch.cuda.synchronize()
    t_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in sev]))
    d_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in sev]))
    # cold pass (untimed for the headline): each step after a scratch fill
    cold = None
    if args.cold_mib > 0:
        scratch = torch.empty(args.cold_mib << 20, dtype=torch.uint8, device=dev)
        cev = [[TimingEvent() for _ in range(2)] for _ in range(args.steps)]
        for i in range(args.steps):
            scratch.fill_(i & 255)
            cev[i][0].record()
            step()
            cev[i][1].record()
        torch.cuda.synchronize()
        ct = np.array([e[0].elapsed_time(e[1]) for e in cev])
        c_med = float(np.median(ct))
        cold = {"flush_mib": args.cold_mib,
                "ms_per_step_median": round(c_med, 4),
                "ms_per_step_p10": round(float(np.percentile(ct, 10)), 4),
                "ms_per_step_p90": round(float(np.percentile(ct, 90)), 4),
                "GB/s": round(nbytes["total"] / (c_med * 1e-3) / 1e9, 1),
                "frac": round(nbytes["total"] / (c_med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "timing": "events around each step; the fill runs before the first event"}
        del scratch
    tokens = Bv * n_q + Bd
    value = tokens / (ms_step / 1e3)

    v_gbs = nbytes["verify"] / (v_ms * 1e-3) / 1e9 if Bv else 0.0
    unit_gbs = nbytes["total"] / (ms_step * 1e-3) / 1e9
    if args.path == "fused":
        # one call does the whole step: its bytes are the step's bytes
        roofline = {
            "kernel": "sss_fused_step (the fused_kernel work-list launch, or for chained whole "
                      "units the verify and select-and-draft launches; split-merge launches "
                      "included in the time)",
            "bound": "hbm",
            "achieved": round(nbytes["total"] / (v_ms * 1e-3) / 1e9, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(nbytes["total"] / (v_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": None,
            "algorithmic_bytes": nbytes["total"],
            "ms": round(v_ms, 4),
        }
    else:
        roofline = {
            "kernel": ("attn_mfma_kernel<verify> (the one launch of sss_verify_attn when units "
                       "run unsplit)" if verify_launches == 1 else
                       "sss_verify_attn (attention, plus the merge / scoring launch when units "
                       "are split)"),
            "bound": "hbm",
            "achieved": round(v_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(v_gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(s.name) if verify_launches == 1 else None,
            "algorithmic_bytes": nbytes["verify"],
            "ms": round(v_ms, 4),
        }
    lens = vb.seq_lens if Bv else db.seq_lens
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
            "verify_splits": vsplits, "draft_splits": args.draft_splits, "path": args.path,
        },
        "roofline": roofline,
        "step_hbm": {
            "algorithmic_bytes": nbytes["total"],
            "GB/s": round(unit_gbs, 1),
            "frac": round(unit_gbs / HBM_PEAK_GBS, 4),
            # K and V alone (every verified token once, every drafted token once)
            "kv_bytes": nbytes["verify_kv"] + nbytes["draft_kv"],
            "kv_GB/s": round((nbytes["verify_kv"] + nbytes["draft_kv"]) / (ms_step * 1e-3) / 1e9, 1),
            "kv_frac": round((nbytes["verify_kv"] + nbytes["draft_kv"]) / (ms_step * 1e-3) / 1e9
                             / HBM_PEAK_GBS, 4),
            "verify_ms": round(v_ms, 4), "topk_ms": round(t_ms, 4), "draft_ms": round(d_ms, 4),
            "stage_times": "verify_ms from the timed steps; topk_ms and draft_ms from a "
                           "separate untimed pass with events between the stages",
            "draft_GB/s": (round(nbytes["draft"] / (d_ms * 1e-3) / 1e9, 1)
                           if Bd and args.path == "separate" else None),
        },
    }
    rec["cold"] = cold
    if args.kv_update and Bv:
        rec["kv_update"] = time_kv_update(wl, kv_v, vb, dev, args.steps)
    if args.cpu_sample > 0:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(wl, args.cpu_sample, args.cpu_seconds)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
