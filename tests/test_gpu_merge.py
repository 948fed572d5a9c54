"""attn_state_merge on the GPU against the oracle.  States accumulated over disjoint key ranges
and merged must match the oracle's merge of the oracle's partial states (state level) and the
single-pass attention over all keys (output level).  The 1M-token Mode B workload ("Out-of-Core
Flash Streaming & Speculative Decode (1M Context)", Sec. 4: 64 candidate queries, the whole
context, no causal mask) is run split into 16 key ranges held as the sequences of one state and
merged, and also streamed into one state; both are checked against the oracle on every row."""
import numpy as np
import pytest
import torch

import chunked_flashattention_q8_amd as q8a
import synthetic
from gpu_util import D, assert_close, dev, f16_to_dev, gpu_pack, say

pytestmark = pytest.mark.gpu


def check_state(m, l, o, ref, label):
    """GPU state (device tensors) against an oracle state: same empty rows (bit-untouched zero
    l), m to FP32 accuracy, O/l and m + ln l within the output bounds."""
    m_ref, l_ref, O_ref = ref
    mg, lg = m.cpu().numpy().reshape(-1), l.cpu().numpy().reshape(-1)
    og = o.cpu().numpy().reshape(-1, D)
    empty = np.isneginf(m_ref)
    assert np.array_equal(np.isneginf(mg), empty), label
    assert not lg[empty].any(), label
    ne = ~empty
    assert np.all(np.abs(mg[ne] - m_ref[ne]) <= 1e-5 * np.maximum(1, np.abs(m_ref[ne]))), label
    assert_close(og[ne] / lg[ne, None], mg[ne] + np.log(lg[ne]), O_ref[ne] / l_ref[ne, None],
                 m_ref[ne] + np.log(l_ref[ne]), label)


@pytest.mark.parametrize("causal", [1, 0])
def test_merge_of_disjoint_ranges(orc, causal):
    """Three key ranges accumulated into three states, merged pairwise; with the causal mask
    some rows see nothing of a range (empty in that state) and must come through unchanged."""
    B, H, M, N, q_pos0 = 2, 3, 200, 336, 133
    say("merge case causal", causal)
    q, k, v = synthetic.small_case(B, H, M, N, q_pos0, seed=60 + causal)
    qd, kd, vd = f16_to_dev(q), gpu_pack(k), gpu_pack(v)
    kb, vb = orc.q8_0_pack(k), orc.q8_0_pack(v)
    prob = orc.Problem(q, kb, vb, orc.KV_Q8_0, q_pos0, bool(causal))
    cuts = [0, 96, 252, N]  # chunk starts on 16-byte boundaries; rows 0..118 see no key of
    # [252, 336) when causal
    states, refs = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        m, l, o = q8a.alloc_state(B, H, M)
        st = q8a.attn_state_init(m, l, o, B, H, M, D, q_pos0)
        for s in range(a, b, 64):
            n = min(64, b - s)
            q8a.attn_accumulate_chunk(st, qd, kd.data_ptr() + s * 68, vd.data_ptr() + s * 68,
                                      q8a.KV_Q8_0, s, n, N * 68, H * N * 68, causal)
        states.append((st, (m, l, o)))
        refs.append(orc.attention_chunks(prob, [(a, b - a)]))
    torch.cuda.synchronize()
    if causal:
        assert np.isneginf(refs[2][0]).any()  # the case exercises empty rows
    # merge the last range into the first, then the middle one
    q8a.attn_state_merge(states[0][0], states[2][0])
    torch.cuda.synchronize()
    ref = orc.merge_states(refs[0], refs[2])
    check_state(*states[0][1], ref, "merge 0+2")
    q8a.attn_state_merge(states[0][0], states[1][0])
    out = torch.empty((B, H, M, D), dtype=torch.float16, device=dev())
    lse = torch.empty((B, H, M), dtype=torch.float32, device=dev())
    q8a.attn_finalize(states[0][0], out, lse)
    torch.cuda.synchronize()
    check_state(*states[0][1], orc.merge_states(ref, refs[1]), "merge 0+2+1")
    O_ref, lse_ref = orc.attention(prob)
    assert_close(out.float().cpu().numpy().reshape(-1, D), lse.cpu().numpy().reshape(-1),
                 O_ref, lse_ref, "merged output")


def test_merge_into_an_empty_state_copies(orc):
    B, H, M, N = 1, 2, 64, 128
    q, k, v = synthetic.small_case(B, H, M, N, 0, seed=9)
    qd, kd, vd = f16_to_dev(q), gpu_pack(k), gpu_pack(v)
    m0, l0, o0 = q8a.alloc_state(B, H, M)
    empty = q8a.attn_state_init(m0, l0, o0, B, H, M, D, 0)
    m1, l1, o1 = q8a.alloc_state(B, H, M)
    full = q8a.attn_state_init(m1, l1, o1, B, H, M, D, 0)
    q8a.attn_accumulate_chunk(full, qd, kd, vd, q8a.KV_Q8_0, 0, N, N * 68, H * N * 68, 1)
    torch.cuda.synchronize()
    o0.fill_(float("nan"))  # O of an empty row is never read
    q8a.attn_state_merge(empty, full)
    torch.cuda.synchronize()
    assert torch.equal(m0, m1) and torch.equal(l0, l1) and torch.equal(o0, o1)
    # and merging an empty state changes nothing
    m2, l2, o2 = q8a.alloc_state(B, H, M)
    empty2 = q8a.attn_state_init(m2, l2, o2, B, H, M, D, 0)
    before = [t.clone() for t in (m1, l1, o1)]
    q8a.attn_state_merge(full, empty2)
    torch.cuda.synchronize()
    for a, b in zip(before, (m1, l1, o1)):
        assert torch.equal(a, b)


def build_burst_cache(orc, w):
    """Q8_0 K/V of the 1M-token Mode B workload: resident on the device [C, 1, H, chunk, 68],
    chunk-major in pinned host memory, and [1, H, N, 68] for the oracle; the GPU pack is checked
    bytewise against the oracle's."""
    H, C, chunk = w.H, w.n_chunks, w.chunk
    kd = torch.empty((C, 1, H, chunk, 68), dtype=torch.uint8, device=dev())
    vd = torch.empty_like(kd)
    kh = torch.empty(kd.shape, dtype=torch.uint8, pin_memory=True)
    vh = torch.empty(kd.shape, dtype=torch.uint8, pin_memory=True)
    k_orc = np.empty((1, H, w.N, 68), dtype=np.uint8)
    v_orc = np.empty((1, H, w.N, 68), dtype=np.uint8)
    for c in range(C):
        k, v = synthetic.gen_kv_chunk(w, c)
        kb, vb = orc.q8_0_pack(k), orc.q8_0_pack(v)
        kd[c, 0] = gpu_pack(k)
        vd[c, 0] = gpu_pack(v)
        kg, vg = kd[c, 0].cpu(), vd[c, 0].cpu()
        assert np.array_equal(kg.numpy(), kb) and np.array_equal(vg.numpy(), vb), c
        kh[c, 0].copy_(kg)
        vh[c, 0].copy_(vg)
        k_orc[0, :, c * chunk:(c + 1) * chunk] = kb
        v_orc[0, :, c * chunk:(c + 1) * chunk] = vb
        if c % 16 == 0:
            say("packed chunk", c, "of", C)
    return kd, vd, kh, vh, k_orc, v_orc


@pytest.mark.timeout(900)
def test_burst_verify_1m_split_and_streamed(orc):
    w = synthetic.WORKLOADS[5]
    H, M, chunk, C = w.H, w.M, w.chunk, w.n_chunks
    kd, vd, kh, vh, k_orc, v_orc = build_burst_cache(orc, w)
    q = synthetic.gen_q(w)
    qd = f16_to_dev(q)
    rb = H * chunk * 68  # bytes of one chunk of one tensor (B = 1)

    # split: 16 consecutive key ranges held as the 16 "sequences" of one state (the queries
    # repeated, the sequence stride stepping from one range to the next), so each chunk call
    # covers all ranges; then the sequence blocks are merged pairwise into sequence 0
    S = 16
    per = C // S
    say("split over", S, "key ranges")
    qrep = qd.expand(S, H, M, D).contiguous()
    m, l, o = q8a.alloc_state(S, H, M)
    st = q8a.attn_state_init(m, l, o, S, H, M, D, w.q_pos0)
    for c in range(per):
        q8a.attn_accumulate_chunk(st, qrep, kd[c].data_ptr(), vd[c].data_ptr(), q8a.KV_Q8_0,
                                  c * chunk, chunk, chunk * 68, per * rb, 0)
    n = S
    while n > 1:
        n //= 2
        q8a.attn_state_merge(q8a.sub_state(st, 0, n), q8a.sub_state(st, n, n))
    out = torch.empty((1, H, M, D), dtype=torch.float16, device=dev())
    lse = torch.empty((1, H, M), dtype=torch.float32, device=dev())
    q8a.attn_finalize(q8a.sub_state(st, 0, 1), out, lse)
    torch.cuda.synchronize()

    # streamed into one state through two device slots
    say("streamed")
    m1, l1, o1 = q8a.alloc_state(1, H, M)
    st1 = q8a.attn_state_init(m1, l1, o1, 1, H, M, D, w.q_pos0)
    slots_k = [torch.empty(rb, dtype=torch.uint8, device=dev()) for _ in range(2)]
    slots_v = [torch.empty(rb, dtype=torch.uint8, device=dev()) for _ in range(2)]
    q8a.attn_accumulate_stream(st1, qd, kh, vh, q8a.KV_Q8_0, w.N, chunk, slots_k, slots_v, 0,
                               torch.cuda.current_stream(), torch.cuda.Stream())
    out1 = torch.empty_like(out)
    lse1 = torch.empty_like(lse)
    q8a.attn_finalize(st1, out1, lse1)
    torch.cuda.synchronize()

    say("oracle on all", H * M, "rows over", w.N, "keys")
    prob = orc.Problem(q, k_orc, v_orc, orc.KV_Q8_0, w.q_pos0, False)
    O_ref, lse_ref = orc.attention(prob)
    for o_, l_, label in ((out, lse, "split + merge"), (out1, lse1, "streamed")):
        assert_close(o_.float().cpu().numpy().reshape(-1, D), l_.cpu().numpy().reshape(-1),
                     O_ref, lse_ref, "burst_verify_1m " + label)
