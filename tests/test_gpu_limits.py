"""Sizes at the edges of what the boundary accepts, against the oracle: byte offsets past 4 GiB
between heads (64-bit head and sequence bases, 32-bit offsets inside a head's chunk), a grid of
4096 (sequence, head) pairs, 16,384 query rows (64 query workgroups per head), and one chunk call
of 262,144 keys (a 4096-tile loop; with N(0, 1) inputs its reference maximum rarely moves -- the
rescale branch itself is exercised by test_gpu_hard.py's constructed inputs)."""
import numpy as np
import pytest
import torch

import chunked_flashattention_q8_amd as q8a
import synthetic
from gpu_util import D, assert_close, dev, f16_to_dev, gpu_pack, prefill, say

pytestmark = pytest.mark.gpu


def oracle_check(orc, q, k, v, q_pos0, out, lse, label, causal=True):
    kb, vb = orc.q8_0_pack(k), orc.q8_0_pack(v)
    prob = orc.Problem(q, kb, vb, orc.KV_Q8_0, q_pos0, causal)
    O_ref, lse_ref = orc.attention(prob)
    assert_close(out.float().cpu().numpy().reshape(-1, D), lse.cpu().numpy().reshape(-1),
                 O_ref, lse_ref, label)
    return kb, vb


@pytest.mark.timeout(300)
def test_head_stride_past_4_gib(orc):
    B, H, M, N, q_pos0 = 2, 2, 96, 300, 204
    hs = (4_500_000_000 // 16) * 16          # 4.19 GiB between heads
    ss = 2 * hs + 1024 * 16                  # sequences outside heads
    n_bytes = (B - 1) * ss + (H - 1) * hs + N * 68 + 16
    say("cache of", n_bytes / 2**30, "GiB per tensor")
    q, k, v = synthetic.small_case(B, H, M, N, q_pos0, seed=41)
    qd = f16_to_dev(q)
    kp, vp = gpu_pack(k), gpu_pack(v)        # [B, H, N, 68]
    kc = torch.empty(n_bytes, dtype=torch.uint8, device=dev())
    vc = torch.empty_like(kc)
    for b in range(B):
        for h in range(H):
            o = b * ss + h * hs
            kc[o:o + N * 68] = kp[b, h].reshape(-1)
            vc[o:o + N * 68] = vp[b, h].reshape(-1)
    m, l, o_ = q8a.alloc_state(B, H, M)
    st = q8a.attn_state_init(m, l, o_, B, H, M, D, q_pos0)
    for s in range(0, N, 100):
        n = min(100, N - s)
        q8a.attn_accumulate_chunk(st, qd, kc.data_ptr() + s * 68, vc.data_ptr() + s * 68,
                                  q8a.KV_Q8_0, s, n, hs, ss, 1)
    out = torch.empty((B, H, M, D), dtype=torch.float16, device=dev())
    lse = torch.empty((B, H, M), dtype=torch.float32, device=dev())
    q8a.attn_finalize(st, out, lse)
    torch.cuda.synchronize()
    del kc, vc
    oracle_check(orc, q, k, v, q_pos0, out, lse, "head stride past 4 GiB")


@pytest.mark.timeout(300)
def test_4096_heads(orc):
    B, H, M, N, q_pos0 = 16, 256, 40, 72, 32
    say("grid of", B * H, "heads")
    q, k, v = synthetic.small_case(B, H, M, N, q_pos0, seed=42)
    out, lse, _ = prefill(f16_to_dev(q), gpu_pack(k), gpu_pack(v), q8a.KV_Q8_0, B, H, M, N,
                          q_pos0, [(0, 36), (36, 36)])
    oracle_check(orc, q, k, v, q_pos0, out, lse, "4096 heads")


@pytest.mark.timeout(300)
def test_16384_query_rows(orc):
    B, H, M, N, q_pos0 = 1, 1, 16384, 16384, 0
    say("M =", M)
    q, k, v = synthetic.small_case(B, H, M, N, q_pos0, seed=43)
    out, lse, _ = prefill(f16_to_dev(q), gpu_pack(k), gpu_pack(v), q8a.KV_Q8_0, B, H, M, N,
                          q_pos0, [(s, 4096) for s in range(0, N, 4096)])
    oracle_check(orc, q, k, v, q_pos0, out, lse, "16384 query rows")


@pytest.mark.timeout(300)
def test_one_call_of_262144_keys(orc):
    B, H, M, N = 1, 2, 256, 262144
    q_pos0 = N - M                           # the last rows: every key visible to most of them
    say("one chunk of", N, "keys")
    q, k, v = synthetic.small_case(B, H, M, N, q_pos0, seed=44)
    out, lse, _ = prefill(f16_to_dev(q), gpu_pack(k), gpu_pack(v), q8a.KV_Q8_0, B, H, M, N,
                          q_pos0, [(0, N)])
    oracle_check(orc, q, k, v, q_pos0, out, lse, "262144 keys in one call")


@pytest.mark.timeout(300)
def test_resume_with_empty_rows_past_2_23(orc):
    """2^23 + 256 query rows of one head, O filled with NaN.  The first chunk (keys 2^23 + 100
    ..) reaches only the last rows; the second (keys 0 .. 63) reaches every row, so the rows
    still empty resume from their state with the past-the-end loads of their l and O, which
    must read 0 even where a head's O spans more than 2 GiB."""
    M = (1 << 23) + 256
    q_pos0 = 0
    say("rows", M)
    q = synthetic.to_f16_bits(synthetic.randn((1, 1, M, D), 451))
    _, k, v = synthetic.small_case(1, 1, 1, 128, 0, seed=45)
    kb, vb = orc.q8_0_pack(k), orc.q8_0_pack(v)   # keys 0..63 -> chunk B, 64..127 -> chunk A
    qd = f16_to_dev(q)
    kd = torch.from_numpy(kb).to(dev())
    vd = torch.from_numpy(vb).to(dev())
    m, l, o = q8a.alloc_state(1, 1, M)
    o.fill_(float("nan"))
    st = q8a.attn_state_init(m, l, o, 1, 1, M, D, q_pos0)
    a_pos = (1 << 23) + 100
    q8a.attn_accumulate_chunk(st, qd, kd.data_ptr() + 64 * 68, vd.data_ptr() + 64 * 68,
                              q8a.KV_Q8_0, a_pos, 64, 128 * 68, 128 * 68, 1)
    q8a.attn_accumulate_chunk(st, qd, kd.data_ptr(), vd.data_ptr(), q8a.KV_Q8_0, 0, 64,
                              128 * 68, 128 * 68, 1)
    out = torch.empty((1, 1, M, D), dtype=torch.float16, device=dev())
    lse = torch.empty((1, 1, M), dtype=torch.float32, device=dev())
    q8a.attn_finalize(st, out, lse)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(lse).all())
    # oracle on sampled rows: the keys are chunk B (positions 0..63) and chunk A (positions
    # a_pos .. a_pos + 63), i.e. key j of kb[:, :, 64 + j] sits at position a_pos + j
    rows = np.concatenate([np.arange(0, 70), np.arange((1 << 23) - 8, (1 << 23) + 8),
                           np.arange(M - 160, M)])
    qs = q[:, :, rows]
    O_ref = np.empty((len(rows), D))
    lse_ref = np.empty(len(rows))
    kq = kb[0, 0].astype(np.uint8)
    for i, r in enumerate(rows):
        # keys this row sees: B keys 0..min(r, 63), A keys at a_pos + j <= r
        vis_b = np.arange(0, min(r, 63) + 1)
        vis_a = 64 + np.arange(0, max(0, min(63, r - a_pos) + 1)) if r >= a_pos else np.arange(0)
        idx = np.concatenate([vis_b, vis_a]).astype(np.int64)
        prob = orc.Problem(qs[:, :, i:i + 1], kb[:, :, idx], vb[:, :, idx], orc.KV_Q8_0,
                           len(idx) - 1, False)
        Oi, li = orc.attention(prob)
        O_ref[i], lse_ref[i] = Oi[0], li[0]
    got = out[0, 0].float().cpu().numpy()[rows]
    assert_close(got, lse[0, 0].cpu().numpy()[rows], O_ref, lse_ref, "rows past 2^23")
