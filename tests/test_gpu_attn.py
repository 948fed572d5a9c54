"""GPU chunked causal attention against the FP64 oracle, element by element, through the C ABI.

Small cases span several query workgroups and 64-key tiles and end in ragged tails (query
counts that leave partial wavefronts, chunk lengths whose byte size is not a multiple of 16);
the edge cases are a single key, chunks no query can see, non-causal chunks, shuffled chunk
order, checkpoint/resume and the empty state."""
import numpy as np
import pytest
import torch

import chunked_flashattention_q8_amd as q8a
import synthetic
from gpu_util import (D, assert_close, dev, f16_to_dev, gpu_pack, metrics, prefill, rows_of,
                      say)

pytestmark = pytest.mark.gpu


def setup_case(orc, B, H, M, N, q_pos0, seed, kv_dtype=q8a.KV_Q8_0):
    q, k, v = synthetic.small_case(B, H, M, N, q_pos0, seed)
    qd = f16_to_dev(q)
    if kv_dtype == q8a.KV_Q8_0:
        kd, vd = gpu_pack(k), gpu_pack(v)
        kb, vb = orc.q8_0_pack(k), orc.q8_0_pack(v)
        torch.cuda.synchronize()
        assert np.array_equal(kd.cpu().numpy(), kb) and np.array_equal(vd.cpu().numpy(), vb)
        prob = orc.Problem(q, kb, vb, orc.KV_Q8_0, q_pos0)
    else:
        kb, vb = synthetic.to_f16_bits(k), synthetic.to_f16_bits(v)
        kd, vd = f16_to_dev(kb), f16_to_dev(vb)
        prob = orc.Problem(q, kb, vb, orc.KV_F16, q_pos0)
    return prob, qd, kd, vd


def chunk_list(N, bc):
    return [(s, min(bc, N - s)) for s in range(0, N, bc)]


CASES = [
    # B, H, M, N, q_pos0, chunk, causal.  The cache holds N rounded up to a multiple of 4 keys
    # (so head strides are 16-byte multiples); the chunks cover keys [0, N).
    (1, 2, 200, 200, 0, 64, 1),       # ragged query tile and wavefront, ragged last tile
    (2, 3, 130, 333, 203, 100, 1),    # last chunk of 33 keys: 2244 bytes, not a 16-multiple
    (1, 1, 1, 1, 0, 1, 1),            # one query, one key
    (1, 2, 31, 97, 66, 12, 1),        # fewer rows than a wavefront, many small chunks
    (1, 2, 64, 1000, 936, 1000, 1),   # one chunk, queries at the end of a longer cache
    (1, 2, 100, 152, 0, 52, 0),       # non-causal
    (1, 2, 40, 500, 0, 128, 1),       # chunks after every query position: no row touched
    (3, 1, 384, 384, 0, 384, 1),      # three sequences, full diagonal in one chunk
    # up to 64 rows: the keys of every tile are split between wavefront pairs
    (2, 2, 33, 290, 257, 64, 1),      # second 32-row block holds one row
    (1, 3, 64, 640, 0, 160, 0),       # non-causal, state resumed over four chunks
    (2, 1, 57, 1200, 1150, 300, 1),   # diagonal in the last chunk, ragged last tile
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_small_cases(orc, case, rows_per_workgroup):
    B, H, M, N, q_pos0, bc, causal = case
    say("case", case, "rows per workgroup", rows_per_workgroup)
    n_alloc = (N + 3) // 4 * 4
    assert causal or n_alloc == N  # without the mask every allocated key would be visible
    prob, qd, kd, vd = setup_case(orc, B, H, M, n_alloc, q_pos0, seed=sum(case))
    prob.causal = bool(causal)
    out, lse, _ = prefill(qd, kd, vd, q8a.KV_Q8_0, B, H, M, n_alloc, q_pos0,
                          chunk_list(N, bc), causal)
    O_ref, lse_ref = orc.attention(prob)
    assert_close(out.float().cpu().numpy().reshape(-1, D), lse.cpu().numpy().reshape(-1),
                 O_ref, lse_ref, str(case))


@pytest.mark.parametrize("case", [(1, 2, 200, 200, 0, 64), (2, 3, 300, 520, 220, 100),
                                  (1, 4, 520, 520, 0, 520), (2, 2, 130, 333, 203, 100)])
def test_row_forms_agree_bit_for_bit(orc, case):
    """128- and 256-row workgroups compute every row the same way: the same state and output
    bits."""
    import gpu_util
    B, H, M, N, q_pos0, bc = case
    n_alloc = (N + 3) // 4 * 4
    prob, qd, kd, vd = setup_case(orc, B, H, M, n_alloc, q_pos0, seed=sum(case))
    res = {}
    for rows in ("128", "256"):
        say("case", case, "rows per workgroup", rows)
        gpu_util.TILE_FORM[0] = gpu_util.FORMS[rows]
        try:
            out, lse, (m, l, o) = prefill(qd, kd, vd, q8a.KV_Q8_0, B, H, M, n_alloc, q_pos0,
                                          chunk_list(N, bc))
        finally:
            gpu_util.TILE_FORM[0] = gpu_util.FORMS["auto"]
        mm = m.cpu().numpy().reshape(-1)
        ne = ~np.isneginf(mm)
        res[rows] = (out.cpu().numpy().view(np.uint16), lse.cpu().numpy().view(np.uint32),
                     mm.view(np.uint32), l.cpu().numpy().view(np.uint32),
                     o.cpu().numpy().reshape(-1, D)[ne].view(np.uint32))
    for a, b in zip(res["128"], res["256"]):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("M", [150, 50])
def test_fp16_kv_small(orc, M, rows_per_workgroup):
    B, H, N, q_pos0 = 2, 2, 260, 110
    say("fp16 kv, M", M, "rows per workgroup", rows_per_workgroup)
    prob, qd, kd, vd = setup_case(orc, B, H, M, N, q_pos0, seed=77, kv_dtype=q8a.KV_F16)
    out, lse, _ = prefill(qd, kd, vd, q8a.KV_F16, B, H, M, N, q_pos0, chunk_list(N, 80))
    O_ref, lse_ref = orc.attention(prob)
    assert_close(out.float().cpu().numpy().reshape(-1, D), lse.cpu().numpy().reshape(-1),
                 O_ref, lse_ref, "fp16")


def test_state_after_every_chunk(orc):
    """After each call the state matches the oracle's recurrence state: same non-empty rows,
    m to FP32 accuracy, and the running softmax O/l and m + ln l within the output bounds."""
    B, H, M, N, q_pos0, bc = 1, 4, 256, 256, 0, 64
    prob, qd, kd, vd = setup_case(orc, B, H, M, N, q_pos0, seed=100)
    ref = [None]

    def on_state(s, n, m, l, o):
        ref[0] = orc.attention_chunks(prob, [(s, n)], state=ref[0])
        m_ref, l_ref, O_ref = ref[0]
        mg, lg = m.cpu().numpy().reshape(-1), l.cpu().numpy().reshape(-1)
        og = o.cpu().numpy().reshape(-1, D)
        empty = np.isneginf(m_ref)
        assert np.array_equal(np.isneginf(mg), empty)
        assert not lg[empty].any()
        ne = ~empty
        assert np.all(np.abs(mg[ne] - m_ref[ne]) <= 1e-5 * np.maximum(1, np.abs(m_ref[ne])))
        assert_close(og[ne] / lg[ne, None], mg[ne] + np.log(lg[ne]),
                     O_ref[ne] / l_ref[ne, None], m_ref[ne] + np.log(l_ref[ne]),
                     "state after chunk at %d" % s)

    prefill(qd, kd, vd, q8a.KV_Q8_0, B, H, M, N, q_pos0, chunk_list(N, bc), on_state=on_state)


def test_rows_without_visible_keys_are_untouched(orc):
    B, H, M, N, q_pos0 = 1, 2, 256, 512, 0
    prob, qd, kd, vd = setup_case(orc, B, H, M, N, q_pos0, seed=5)
    m, l, o = q8a.alloc_state(B, H, M)
    st = q8a.attn_state_init(m, l, o, B, H, M, D, q_pos0)
    q8a.attn_accumulate_chunk(st, qd, kd, vd, 0, 0, 192, N * 68, H * N * 68, 1)
    torch.cuda.synchronize()
    before = [t.clone() for t in (m, l, o)]
    # keys 256..511 come after every query position
    q8a.attn_accumulate_chunk(st, qd, kd.data_ptr() + 256 * 68, vd.data_ptr() + 256 * 68, 0,
                              256, 256, N * 68, H * N * 68, 1)
    torch.cuda.synchronize()
    for a, b in zip(before, (m, l, o)):
        assert torch.equal(a, b)
    # keys 192..255: rows 0..191 see none of them and stay bit-identical
    q8a.attn_accumulate_chunk(st, qd, kd.data_ptr() + 192 * 68, vd.data_ptr() + 192 * 68, 0,
                              192, 64, N * 68, H * N * 68, 1)
    torch.cuda.synchronize()
    assert torch.equal(before[0][..., :192], m[..., :192])
    assert torch.equal(before[2][..., :192, :], o[..., :192, :])
    assert not torch.equal(before[2][..., 192:, :], o[..., 192:, :])


def test_shuffled_chunk_order(orc):
    B, H, M, N, q_pos0 = 1, 3, 300, 640, 340
    prob, qd, kd, vd = setup_case(orc, B, H, M, N, q_pos0, seed=9)
    chunks = chunk_list(N, 64)
    order = np.random.default_rng(1).permutation(len(chunks))
    out, lse, _ = prefill(qd, kd, vd, 0, B, H, M, N, q_pos0, [chunks[i] for i in order])
    O_ref, lse_ref = orc.attention(prob)
    assert_close(out.float().cpu().numpy().reshape(-1, D), lse.cpu().numpy().reshape(-1),
                 O_ref, lse_ref, "shuffled")


def test_deterministic_and_resumable(orc):
    B, H, M, N, q_pos0 = 2, 2, 256, 512, 256
    prob, qd, kd, vd = setup_case(orc, B, H, M, N, q_pos0, seed=21)
    chunks = chunk_list(N, 128)
    out1, lse1, _ = prefill(qd, kd, vd, 0, B, H, M, N, q_pos0, chunks)
    out2, lse2, _ = prefill(qd, kd, vd, 0, B, H, M, N, q_pos0, chunks)
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)
    # checkpoint after two chunks, clobber the device state, restore, finish
    m, l, o = q8a.alloc_state(B, H, M)
    st = q8a.attn_state_init(m, l, o, B, H, M, D, q_pos0)
    prefill(qd, kd, vd, 0, B, H, M, N, q_pos0, chunks[:2], state=(st, (m, l, o)))
    saved = [t.cpu() for t in (m, l, o)]
    for t in (m, l, o):
        t.fill_(float("nan"))
    for t, s in zip((m, l, o), saved):
        t.copy_(s)
    out3, lse3, _ = prefill(qd, kd, vd, 0, B, H, M, N, q_pos0, chunks[2:], state=(st, (m, l, o)))
    assert torch.equal(out1, out3) and torch.equal(lse1, lse3)


def test_empty_state_finalize():
    B, H, M = 1, 2, 100
    m, l, o = q8a.alloc_state(B, H, M)
    o.fill_(float("nan"))  # an empty row's O is never read
    st = q8a.attn_state_init(m, l, o, B, H, M, D, 0)
    out = torch.full((B, H, M, D), 7.0, dtype=torch.float16, device="cuda")
    lse = torch.zeros((B, H, M), dtype=torch.float32, device="cuda")
    q8a.attn_finalize(st, out, lse)
    torch.cuda.synchronize()
    assert not out.any()
    assert torch.all(torch.isneginf(lse))


# ---------------------------------------------------------------- the workloads' own shapes

def run_workload(orc, wid, kv_dtype=q8a.KV_Q8_0, chunk=None, rows_per_head=None, append=False):
    w = synthetic.WORKLOADS[wid]
    say("workload", w.name, "dtype", kv_dtype, "chunk", chunk or w.chunk)
    q = synthetic.gen_q(w)
    k, v = synthetic.gen_kv(w)
    qd = f16_to_dev(q)
    if kv_dtype == q8a.KV_Q8_0:
        kb, vb = orc.q8_0_pack(k), orc.q8_0_pack(v)
        kd, vd = gpu_pack(k), gpu_pack(v)
        torch.cuda.synchronize()
        assert np.array_equal(kd.cpu().numpy(), kb) and np.array_equal(vd.cpu().numpy(), vb)
        prob = orc.Problem(q, kb, vb, orc.KV_Q8_0, w.q_pos0)
    else:
        kb, vb = synthetic.to_f16_bits(k), synthetic.to_f16_bits(v)
        kd, vd = f16_to_dev(kb), f16_to_dev(vb)
        prob = orc.Problem(q, kb, vb, orc.KV_F16, w.q_pos0)
    bc = chunk or w.chunk
    chunks = [(s, min(bc, w.N - s)) for s in range(0, w.N, bc)]
    if append:
        # the tokens at positions >= q_pos0 arrive with the queries: their cache rows start
        # out as junk and are written by attn_append_chunk from the FP32 values
        assert w.B == 1 and chunks[-1][0] == w.q_pos0
        kd[:, :, w.q_pos0:] = 0xA5
        vd[:, :, w.q_pos0:] = 0xA5
        chunks = chunks[:-1]
        m, l, o = q8a.alloc_state(w.B, w.H, w.M)
        st = q8a.attn_state_init(m, l, o, w.B, w.H, w.M, D, w.q_pos0)
        prefill(qd, kd, vd, kv_dtype, w.B, w.H, w.M, w.N, w.q_pos0, chunks,
                state=(st, (m, l, o)), finalize=False)
        kn = torch.from_numpy(np.ascontiguousarray(k[:, :, w.q_pos0:])).to(dev())
        vn = torch.from_numpy(np.ascontiguousarray(v[:, :, w.q_pos0:])).to(dev())
        say("append", w.N - w.q_pos0, "tokens")
        q8a.attn_append_chunk(st, qd, kn, vn, kd.data_ptr() + w.q_pos0 * 68,
                              vd.data_ptr() + w.q_pos0 * 68, w.q_pos0, w.N - w.q_pos0,
                              w.N * 68, w.H * w.N * 68, 1)
        out = torch.empty((w.B, w.H, w.M, D), dtype=torch.float16, device=dev())
        lse = torch.empty((w.B, w.H, w.M), dtype=torch.float32, device=dev())
        q8a.attn_finalize(st, out, lse)
        torch.cuda.synchronize()
        assert np.array_equal(kd[:, :, w.q_pos0:].cpu().numpy(), kb[:, :, w.q_pos0:])
        assert np.array_equal(vd[:, :, w.q_pos0:].cpu().numpy(), vb[:, :, w.q_pos0:])
        del kn, vn
    else:
        out, lse, _ = prefill(qd, kd, vd, kv_dtype, w.B, w.H, w.M, w.N, w.q_pos0, chunks)
    del k, v
    rows = synthetic.sample_rows(w, rows_per_head)
    O_ref, lse_ref = orc.attention(prob, rows)
    return assert_close(rows_of(out, rows, D), rows_of(lse, rows), O_ref, lse_ref, w.name)


def test_workload_tiny(orc):
    run_workload(orc, 0)


def test_workload_incore_m2048(orc):
    run_workload(orc, 1)


@pytest.mark.timeout(300)
def test_workload_batch8_q8_0(orc):
    run_workload(orc, 2)


@pytest.mark.timeout(300)
def test_workload_batch8_f16(orc):
    run_workload(orc, 2, kv_dtype=q8a.KV_F16)


@pytest.mark.timeout(300)
def test_workload_batch8_one_chunk(orc):
    run_workload(orc, 2, chunk=2048)


@pytest.mark.timeout(300)
def test_workload_append_133k(orc):
    """The 131,072 cached tokens through attn_accumulate_chunk, the 2048 appended tokens (the
    queries' own positions) through attn_append_chunk from FP32."""
    run_workload(orc, 3, append=True)


# Chunks of 512 keys and more: in the 256-row form the state's O of resumed rows reaches the
# kernel spread over its first tiles (8 KiB blocks of 32 rows through LDS); exactly 8 tiles (the
# last block is added after the loop) and more than 8; ragged query tiles; states whose rows are
# partly empty (a chunk after some query positions first); chunk orders that resume rows from a
# later chunk.
BIG_CHUNKS = [
    # B, H, M, N, q_pos0, chunk, order of the chunks (indices into the ascending list)
    (1, 2, 300, 1600, 1300, 512, None),         # 8-tile calls, the last call one tile
    (2, 1, 260, 2000, 1740, 640, None),         # 10-tile calls
    (1, 2, 600, 1024, 0, 512, (1, 0)),          # rows 512..599 resumed, rows 0..511 fresh
    (1, 1, 256, 1536, 1024, 512, (2, 0, 1)),    # the diagonal chunk first
]


@pytest.mark.parametrize("case", BIG_CHUNKS, ids=[str(c) for c in BIG_CHUNKS])
def test_big_chunks(orc, case, rows_per_workgroup):
    B, H, M, N, q_pos0, bc, order = case
    say("big chunks", case, "rows per workgroup", rows_per_workgroup)
    prob, qd, kd, vd = setup_case(orc, B, H, M, N, q_pos0, seed=sum(case[:6]))
    chunks = chunk_list(N, bc)
    if order is not None:
        chunks = [chunks[i] for i in order]
    out, lse, _ = prefill(qd, kd, vd, q8a.KV_Q8_0, B, H, M, N, q_pos0, chunks)
    O_ref, lse_ref = orc.attention(prob)
    assert_close(out.float().cpu().numpy().reshape(-1, D), lse.cpu().numpy().reshape(-1),
                 O_ref, lse_ref, str(case))
