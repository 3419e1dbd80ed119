"""GPU parity of the KV update entry points (sss_kv_write, sss_kv_commit)
against the oracle, through the C ABI: the whole cache compared bit-exactly
after a write, the lengths bit-exactly after a commit, and one speculative
round trip (write the new positions, verify, commit, write and verify the
next step) against the oracle's verify on its own updated cache."""
import numpy as np
import pytest
import torch

import harness as H
import oracle
from sparse_self_speculative_sss_amd import workload as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


def host(t):
    return t.detach().cpu()


def as_bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


CASES = [
    ("bf16_d128_p16", "qwen3_8b_layer_b16_l4096", dict(B=3, L=200)),
    ("bf16_d64_p16", "decode_b128_l8192", dict(B=2, L=300, d=64)),
    ("bf16_p64", "longctx_b4_l128k", dict(B=2, L=500)),
    ("f32_d64", "tiny_fp32_b1_l512", dict(B=2, L=100)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_kv_write_bit_exact(case):
    cid, name, kw = case
    wl = W.make(name, seed=41, device=DEV, **kw)
    vb = wl.verify
    B = vb.B
    hkv, d = wl.shape.Hkv, wl.shape.d
    n_new = wl.shape.n_q
    g = torch.Generator(device=DEV)
    g.manual_seed(7)
    k_new = torch.randn((B, n_new, hkv, d), generator=g, device=DEV).to(wl.k_cache.dtype)
    v_new = torch.randn((B, n_new, hkv, d), generator=g, device=DEV).to(wl.k_cache.dtype)
    lens = vb.seq_lens.cpu().numpy()
    # each request's last n_new positions; the last request starts past the
    # end of its table row and the first before position 0 (those rows are
    # skipped)
    pos0 = (lens - n_new).astype(np.int32)
    if B >= 2:
        pos0[-1] = vb.page_table.shape[1] * wl.shape.page_size
        pos0[0] = -2
    pos0_t = torch.from_numpy(pos0).to(DEV)
    ref_k, ref_v = oracle.kv_write(host(wl.k_cache).numpy() if wl.k_cache.dtype == torch.float32
                                   else host(wl.k_cache).float().numpy(),
                                   host(wl.v_cache).float().numpy(), vb.page_table.cpu().numpy(),
                                   host(k_new).float().numpy(), host(v_new).float().numpy(), pos0)
    kv = H.kv_of(wl, vb)
    print(f"[kv_write] {cid}", flush=True)
    H.sss().kv_write(kv, k_new, v_new, pos0_t)
    torch.cuda.synchronize()
    got_k = host(wl.k_cache).float().numpy()
    got_v = host(wl.v_cache).float().numpy()
    assert np.array_equal(got_k, ref_k)
    assert np.array_equal(got_v, ref_v)


def test_kv_write_negative_and_bad_page_skipped():
    wl = W.make("qwen3_8b_layer_b16_l4096", seed=42, device=DEV, B=2, L=64)
    vb = wl.verify
    before_k, before_v = wl.k_cache.clone(), wl.v_cache.clone()
    table = vb.page_table.clone()
    table[1, :] = 10 ** 7                              # no valid page for request 1
    kv = H.sss().paged_kv(wl.k_cache, wl.v_cache, table, vb.seq_lens, vb.max_seq_len)
    k_new = torch.ones((2, 3, wl.shape.Hkv, wl.shape.d), dtype=torch.bfloat16, device=DEV)
    pos0 = torch.tensor([-3, 10], dtype=torch.int32, device=DEV)
    H.sss().kv_write(kv, k_new, k_new, pos0)
    torch.cuda.synchronize()
    assert torch.equal(as_bits(wl.k_cache), as_bits(before_k))
    assert torch.equal(as_bits(wl.v_cache), as_bits(before_v))


def test_kv_commit_bit_exact():
    g = np.random.default_rng(3)
    for n_q in (1, 5, 9):
        lens = g.integers(0, 5000, 300).astype(np.int32)
        keep = g.integers(-3, n_q + 4, 300).astype(np.int32)
        ref = oracle.kv_commit(lens, keep, n_q)
        lt = torch.from_numpy(lens).to(DEV)
        kt = torch.from_numpy(keep).to(DEV)
        out = torch.full_like(lt, -1)
        H.sss().kv_commit(lt, kt, n_q, out)
        H.sss().kv_commit(lt, kt, n_q)                 # in place
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), ref)
        assert np.array_equal(lt.cpu().numpy(), ref)


def test_speculative_round_trip():
    """write the k+1 positions -> verify -> commit -> write the next k+1 on top of the
    kept prefix -> verify: both verifies match the oracle on its own cache."""
    wl = W.make("qwen3_8b_layer_b16_l4096", seed=43, device=DEV, B=3, L=600, sigma="one")
    vb = wl.verify
    s = H.sss()
    B, n_q, hq, d = vb.q.shape
    hkv = wl.shape.Hkv
    g = torch.Generator(device=DEV)
    g.manual_seed(11)
    lens = vb.seq_lens.clone()
    hk = host(wl.k_cache).float().numpy()
    hv = host(wl.v_cache).float().numpy()
    table = vb.page_table.cpu().numpy()
    keep = torch.tensor([1, 3, 5], dtype=torch.int32, device=DEV)
    for step in range(2):
        # the table holds pages for every position this step writes
        assert int(lens.max()) <= vb.page_table.shape[1] * wl.shape.page_size
        k_new = torch.randn((B, n_q, hkv, d), generator=g, device=DEV).to(torch.bfloat16)
        v_new = torch.randn((B, n_q, hkv, d), generator=g, device=DEV).to(torch.bfloat16)
        pos0 = (lens - n_q).to(torch.int32)
        kv = s.paged_kv(wl.k_cache, wl.v_cache, vb.page_table, lens, vb.max_seq_len + n_q)
        s.kv_write(kv, k_new, v_new, pos0)
        hk, hv = oracle.kv_write(hk, hv, table, host(k_new).float().numpy(),
                                 host(v_new).float().numpy(), pos0.cpu().numpy())
        o = torch.empty_like(vb.q)
        lse = torch.empty((B, n_q, hq), device=DEV)
        sc = torch.empty((B, hkv, wl.max_blocks + 8), device=DEV)
        s.verify_attn(kv, vb.q, wl.sm_scale, wl.shape.block_size, wl.max_blocks + 8, o, lse, sc)
        torch.cuda.synchronize()
        L_np = lens.cpu().numpy()
        O_ref, LSE_ref = oracle.verify(W.to_numpy64(vb.q), hk, hv, table, L_np, wl.sm_scale)
        st = H.Stats()
        st.add_o(o.float().cpu().numpy().astype(np.float64), O_ref)
        st.add_lse(lse.cpu().numpy().astype(np.float64), LSE_ref)
        st.check(f"round trip step {step}")
        # accept: keep a prefix of the speculative positions, then the next
        # step's k+1 positions go on top of it
        s.kv_commit(lens, keep, n_q)
        torch.cuda.synchronize()
        lens = lens + n_q
