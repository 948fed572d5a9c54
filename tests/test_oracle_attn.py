"""Pins the oracle's attention to results fixed independently of it:

* torch's CPU scaled_dot_product_attention and logsumexp in float64 (library routines) on the
  same dequantised values, causal mask included;
* closed forms: K = 0 gives uniform weights; the first position sees only key 0;
* 50-digit mpmath brute force on tiny inputs, including very large logits;
* the exactness claim of the chunk recurrence ("Out-of-Core Flash Streaming & Speculative Decode
  (1M Context)", Sec. 3): any chunking and any chunk order give the single-pass result, and the
  state after the first k chunks is the single-pass result over that prefix.
"""
import mpmath
import numpy as np
import pytest
import torch

from synthetic import small_case, to_f16_bits

D = 64


def dequant_np(b):
    """Independent Q8_0 decode with numpy's float16: value = int8 * scale."""
    b = np.asarray(b, dtype=np.uint8)
    blocks = b.reshape(b.shape[:-1] + (-1, 34))
    scale = blocks[..., :2].copy().view(np.float16).astype(np.float64)
    q = blocks[..., 2:].copy().view(np.int8).astype(np.float64)
    return (q * scale).reshape(b.shape[:-1] + (-1,))


def make(orc, B, H, M, N, q_pos0, seed, causal=True, fmt="q8_0", qscale=1.0):
    q, k, v = small_case(B, H, M, N, q_pos0, seed)
    if qscale != 1.0:
        q = to_f16_bits(q.view(np.float16).astype(np.float32) * np.float32(qscale))
    if fmt == "q8_0":
        kb, vb = orc.q8_0_pack(k), orc.q8_0_pack(v)
        kd, vd = dequant_np(kb), dequant_np(vb)
        prob = orc.Problem(q, kb, vb, orc.KV_Q8_0, q_pos0, causal)
    else:
        kb, vb = to_f16_bits(k), to_f16_bits(v)
        kd = kb.view(np.float16).astype(np.float64)
        vd = vb.view(np.float16).astype(np.float64)
        prob = orc.Problem(q, kb, vb, orc.KV_F16, q_pos0, causal)
    qd = q.view(np.float16).astype(np.float64)
    return prob, qd, kd, vd


def mask_for(M, N, q_pos0, causal):
    pos = q_pos0 + np.arange(M)[:, None]
    return (np.arange(N)[None, :] <= pos) if causal else np.ones((M, N), dtype=bool)


def torch_ref(qd, kd, vd, q_pos0, causal):
    M, N = qd.shape[2], kd.shape[2]
    mask = torch.from_numpy(mask_for(M, N, q_pos0, causal))
    q, k, v = (torch.from_numpy(a) for a in (qd, kd, vd))
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)
    s = torch.matmul(q, k.transpose(-1, -2).contiguous()) / 8.0
    s = s.masked_fill(~mask, float("-inf"))
    return o.numpy(), torch.logsumexp(s, dim=-1).numpy(), s.numpy()


@pytest.mark.parametrize("B,H,M,N,q_pos0,causal", [
    (1, 2, 40, 40, 0, True),
    (2, 3, 37, 53, 16, True),
    (1, 2, 19, 70, 3, True),     # queries early in a longer cache: later keys masked
    (2, 1, 33, 29, 5, False),
    (1, 1, 8, 300, 292, True),
])
def test_matches_torch_sdpa(orc, B, H, M, N, q_pos0, causal):
    prob, qd, kd, vd = make(orc, B, H, M, N, q_pos0, seed=B * 100 + N, causal=causal)
    O, lse = orc.attention(prob)
    o_ref, lse_ref, _ = torch_ref(qd, kd, vd, q_pos0, causal)
    np.testing.assert_allclose(O, o_ref.reshape(-1, D), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref.reshape(-1), rtol=1e-14, atol=1e-13)


def test_f16_kv_matches_torch(orc):
    prob, qd, kd, vd = make(orc, 1, 2, 24, 40, 16, seed=5, fmt="f16")
    O, lse = orc.attention(prob)
    o_ref, lse_ref, _ = torch_ref(qd, kd, vd, 16, True)
    np.testing.assert_allclose(O, o_ref.reshape(-1, D), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref.reshape(-1), rtol=1e-14, atol=1e-13)


def test_zero_keys_give_uniform_weights(orc):
    """K = 0 makes every visible logit 0: O_i is the mean of V over keys 0..p_i and
    LSE_i = ln(p_i + 1)."""
    M, N, q_pos0 = 30, 50, 7
    prob, qd, kd, vd = make(orc, 1, 2, M, N, q_pos0, seed=9)
    prob.k = np.zeros_like(prob.k)
    O, lse = orc.attention(prob)
    O = O.reshape(2, M, D)
    lse = lse.reshape(2, M)
    for h in range(2):
        for i in range(M):
            p = q_pos0 + i
            np.testing.assert_allclose(O[h, i], vd[0, h, :p + 1].mean(axis=0), atol=1e-14)
            assert abs(lse[h, i] - np.log(p + 1)) < 1e-14


def test_first_position_sees_only_key_zero(orc):
    prob, qd, kd, vd = make(orc, 1, 3, 4, 16, 0, seed=12)
    O, lse = orc.attention(prob)
    O = O.reshape(3, 4, D)
    for h in range(3):
        assert np.array_equal(O[h, 0], vd[0, h, 0])
        assert abs(lse.reshape(3, 4)[h, 0] - qd[0, h, 0] @ kd[0, h, 0] / 8) < 1e-14


def _mp_attention(qd, kd, vd, q_pos0, causal):
    mpmath.mp.dps = 50
    M, N = qd.shape[0], kd.shape[0]
    outs, lses = [], []
    for i in range(M):
        vis = range(N) if not causal else range(min(q_pos0 + i + 1, N))
        s = [mpmath.fsum(mpmath.mpf(qd[i, t]) * mpmath.mpf(kd[j, t]) for t in range(D)) / 8
             for j in vis]
        w = [mpmath.e ** x for x in s]
        l = mpmath.fsum(w)
        outs.append([float(mpmath.fsum(w[a] * mpmath.mpf(vd[j, t]) for a, j in enumerate(vis))
                           / l) for t in range(D)])
        lses.append(float(mpmath.log(l)))
    return np.array(outs), np.array(lses)


@pytest.mark.parametrize("M,N,q_pos0,causal,qscale", [
    (6, 6, 0, True, 1.0),
    (5, 9, 4, True, 1.0),
    (4, 7, 2, False, 1.0),
    (5, 12, 7, True, 40.0),   # logits of order +-100: alpha << 1, exp underflow
])
def test_mpmath_brute_force(orc, M, N, q_pos0, causal, qscale):
    prob, qd, kd, vd = make(orc, 1, 1, M, N, q_pos0, seed=M * N, causal=causal, qscale=qscale)
    O, lse = orc.attention(prob)
    o_mp, lse_mp = _mp_attention(qd[0, 0], kd[0, 0], vd[0, 0], q_pos0, causal)
    np.testing.assert_allclose(O, o_mp, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_mp, rtol=1e-13, atol=1e-12)
    # the chunk recurrence with one-key chunks reaches the same values
    st = orc.attention_chunks(prob, [(j, 1) for j in range(N)])
    O2, lse2 = orc.finalize(*st)
    np.testing.assert_allclose(O2, o_mp, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse2, lse_mp, rtol=1e-13, atol=1e-12)


@pytest.mark.parametrize("bc", [1, 7, 64, 200])
@pytest.mark.parametrize("shuffle", [False, True])
def test_chunked_equals_single_pass(orc, bc, shuffle):
    M, N, q_pos0 = 48, 200, 152
    prob, qd, kd, vd = make(orc, 2, 2, M, N, q_pos0, seed=31)
    O, lse = orc.attention(prob)
    chunks = [(s, min(bc, N - s)) for s in range(0, N, bc)]
    if shuffle:
        order = np.random.default_rng(bc).permutation(len(chunks))
        chunks = [chunks[i] for i in order]
    O2, lse2 = orc.finalize(*orc.attention_chunks(prob, chunks))
    np.testing.assert_allclose(O2, O, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13, atol=1e-12)


def test_state_after_each_chunk_is_prefix_attention(orc):
    """After chunks 0..k the state holds the single-pass attention over keys [0, (k+1) B_C):
    O / l and m + ln l match it, and m is the largest visible logit of that prefix."""
    M, N, q_pos0, bc = 24, 96, 72, 32
    prob, qd, kd, vd = make(orc, 1, 2, M, N, q_pos0, seed=44)
    state = None
    for c, start in enumerate(range(0, N, bc)):
        state = orc.attention_chunks(prob, [(start, bc)], state=state)
        end = start + bc
        o_ref, lse_ref, s = torch_ref(qd[..., :, :], kd[:, :, :end], vd[:, :, :end], q_pos0,
                                      True)
        O2, lse2 = orc.finalize(*state)
        np.testing.assert_allclose(O2, o_ref.reshape(-1, D), rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse2, lse_ref.reshape(-1), rtol=1e-14, atol=1e-13)
        np.testing.assert_allclose(state[0], s.max(axis=-1).reshape(-1), rtol=0, atol=1e-14)


def test_chunk_without_visible_keys_leaves_state_untouched(orc):
    M, N, q_pos0 = 16, 64, 10
    prob, *_ = make(orc, 1, 1, M, N, q_pos0, seed=3)
    st = orc.attention_chunks(prob, [(0, 32)])
    st2 = orc.attention_chunks(prob, [(32, 32)], state=st)  # keys 32..63 > positions 10..25
    for a, b in zip(st, st2):
        assert np.array_equal(a, b)
    # a fresh state that sees nothing stays empty
    st3 = orc.attention_chunks(prob, [(40, 24)])
    assert np.all(np.isneginf(st3[0])) and not st3[1].any() and not st3[2].any()
    out, lse = orc.finalize(*st3)
    assert not out.any() and np.all(np.isneginf(lse))


@pytest.mark.parametrize("causal", [True, False])
def test_merged_partial_states_equal_attention_over_the_union(orc, causal):
    """Partial states over disjoint key ranges, merged, give the single-pass attention over all
    keys (torch's float64 SDPA), for a split into 2 and into 5 ranges merged in shuffled order;
    rows that see none of a range's keys keep the other state."""
    M, N, q_pos0 = 30, 160, 120
    prob, qd, kd, vd = make(orc, 1, 3, M, N, q_pos0, seed=77, causal=causal)
    o_ref, lse_ref, _ = torch_ref(qd, kd, vd, q_pos0, causal)
    for cuts in ([0, 70, N], [0, 13, 40, 99, 141, N]):
        parts = [orc.attention_chunks(prob, [(a, b - a)]) for a, b in zip(cuts[:-1], cuts[1:])]
        order = np.random.default_rng(len(cuts)).permutation(len(parts))
        st = parts[order[0]]
        for i in order[1:]:
            st = orc.merge_states(st, parts[i])
        O, lse = orc.finalize(*st)
        np.testing.assert_allclose(O, o_ref.reshape(-1, D), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, lse_ref.reshape(-1), rtol=1e-13, atol=1e-12)


def test_merge_with_an_empty_state_is_the_identity(orc):
    M, N, q_pos0 = 12, 64, 20
    prob, *_ = make(orc, 1, 2, M, N, q_pos0, seed=5)
    st = orc.attention_chunks(prob, [(0, 40)])
    empty = orc.init_state(st[0].size, D)
    for a, b in ((st, empty), (empty, st)):
        out = orc.merge_states(a, b)
        for x, y in zip(out, st):
            assert np.array_equal(x, y)
    both = orc.merge_states(empty, empty)
    assert np.all(np.isneginf(both[0])) and not both[1].any() and not both[2].any()
