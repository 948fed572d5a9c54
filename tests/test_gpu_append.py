"""attn_append_chunk (quantise-on-append, "Core Architecture & The 4-Brick Pipeline", Sec. 5:
dynamically quantised block_q8_0 KV) on the GPU: appending FP32 tokens writes exactly the cache
bytes q8_0_pack writes and leaves exactly the state q8_0_pack + attn_accumulate_chunk leaves, and
the output matches the oracle.  Cache layouts: sequences outside heads and heads outside
sequences; chunk lengths that leave a ragged last tile and an odd block count."""
import numpy as np
import pytest
import torch

import chunked_flashattention_q8_amd as q8a
import synthetic
from gpu_util import D, assert_close, dev, f16_to_dev, say

pytestmark = pytest.mark.gpu

FILL = 0xA5


def cache_views(buf, B, H, N, heads_outer):
    """Byte strides of a [B][H][N][68] (or [H][B][N][68]) cache in a flat buffer."""
    row = N * 68
    if heads_outer:
        return B * row, row  # head stride, sequence stride
    return row, H * row


def place(cache, rows, B, H, N, kv_pos0, hs, ss):
    """Write packed rows [B][H][n][68] (numpy) into a flat cache buffer (numpy) in place."""
    n = rows.shape[2]
    for b in range(B):
        for h in range(H):
            o = b * ss + h * hs + kv_pos0 * 68
            cache[o:o + n * 68] = rows[b, h].reshape(-1)


@pytest.mark.parametrize("heads_outer", [False, True])
@pytest.mark.parametrize("B,H,M,N,q_pos0,cut,causal", [
    (2, 3, 200, 400, 200, 252, 1),    # resumed state; new keys 252..399 (148: ragged last tile)
    (1, 2, 64, 97, 64, 64, 1),         # 33 new keys: odd block count per run, one partial tile
    (2, 1, 80, 180, 0, 0, 0),          # everything appended in one call, non-causal
])
def test_append_equals_pack_then_accumulate(orc, heads_outer, B, H, M, N, q_pos0, cut, causal):
    say("append case", B, H, M, N, q_pos0, cut, causal, "heads_outer", heads_outer)
    q, k, v = synthetic.small_case(B, H, M, N, q_pos0, seed=B * 100 + N + cut)
    qd = f16_to_dev(q)
    Na = (N + 3) // 4 * 4 + 8  # allocated keys per (seq, head): row runs start 16-byte aligned
    hs, ss = cache_views(None, B, H, Na, heads_outer)
    total = B * H * Na * 68
    kb, vb = orc.q8_0_pack(k), orc.q8_0_pack(v)
    n_new = N - cut

    def fresh_cache(packed):
        c = np.full(total, FILL, dtype=np.uint8)
        place(c, packed[:, :, :cut], B, H, Na, 0, hs, ss)
        return c

    results = []
    for fused in (True, False):
        kc = torch.from_numpy(fresh_cache(kb)).to(dev())
        vc = torch.from_numpy(fresh_cache(vb)).to(dev())
        m, l, o = q8a.alloc_state(B, H, M)
        st = q8a.attn_state_init(m, l, o, B, H, M, D, q_pos0)
        for s in range(0, cut, 64):  # the cached part: packed rows already in the cache
            n = min(64, cut - s)
            q8a.attn_accumulate_chunk(st, qd, kc.data_ptr() + s * 68, vc.data_ptr() + s * 68,
                                      q8a.KV_Q8_0, s, n, hs, ss, causal)
        kn = torch.from_numpy(np.ascontiguousarray(k[:, :, cut:])).to(dev())
        vn = torch.from_numpy(np.ascontiguousarray(v[:, :, cut:])).to(dev())
        if fused:
            q8a.attn_append_chunk(st, qd, kn, vn, kc.data_ptr() + cut * 68,
                                  vc.data_ptr() + cut * 68, cut, n_new, hs, ss, causal)
        else:  # pack into a contiguous scratch, place the rows, then accumulate them
            kp = torch.empty((B, H, n_new, 68), dtype=torch.uint8, device=dev())
            vp = torch.empty_like(kp)
            q8a.q8_0_pack(kn, kp, B * H * n_new, 64)
            q8a.q8_0_pack(vn, vp, B * H * n_new, 64)
            torch.cuda.synchronize()
            kcn, vcn = kc.cpu().numpy(), vc.cpu().numpy()
            place(kcn, kp.cpu().numpy(), B, H, Na, cut, hs, ss)
            place(vcn, vp.cpu().numpy(), B, H, Na, cut, hs, ss)
            kc.copy_(torch.from_numpy(kcn))
            vc.copy_(torch.from_numpy(vcn))
            q8a.attn_accumulate_chunk(st, qd, kc.data_ptr() + cut * 68,
                                      vc.data_ptr() + cut * 68, q8a.KV_Q8_0, cut, n_new, hs,
                                      ss, causal)
        out = torch.empty((B, H, M, D), dtype=torch.float16, device=dev())
        lse = torch.empty((B, H, M), dtype=torch.float32, device=dev())
        q8a.attn_finalize(st, out, lse)
        torch.cuda.synchronize()
        results.append((kc.cpu().numpy(), vc.cpu().numpy(), m.cpu(), l.cpu(), o.cpu(),
                        out.cpu(), lse.cpu()))
    fused_r, ref_r = results
    # the cache: every appended row equals the oracle's pack, every other byte is untouched
    want_k, want_v = fresh_cache(kb), fresh_cache(vb)
    place(want_k, kb[:, :, cut:], B, H, Na, cut, hs, ss)
    place(want_v, vb[:, :, cut:], B, H, Na, cut, hs, ss)
    assert np.array_equal(fused_r[0], want_k) and np.array_equal(fused_r[1], want_v)
    # the state and the output: bit for bit those of pack + accumulate
    for a, b_ in zip(fused_r[2:], ref_r[2:]):
        assert torch.equal(a, b_)
    prob = orc.Problem(q, kb, vb, orc.KV_Q8_0, q_pos0, bool(causal))
    O_ref, lse_ref = orc.attention(prob)
    assert_close(fused_r[5].float().numpy().reshape(-1, D), fused_r[6].numpy().reshape(-1),
                 O_ref, lse_ref, "append")
