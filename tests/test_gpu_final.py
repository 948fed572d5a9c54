"""attn_accumulate_chunk_final: a causal chunk call that also writes the final output of the rows
whose query position lies inside the chunk.  Against the plain path (attn_accumulate_chunk for
every chunk, then attn_finalize) on the same inputs: the state after the pass is the same bit for
bit, out and lse of every row some chunk completes are the same bit for bit, and the rows no
chunk completes keep what out and lse held before.  The completed rows also meet the oracle at
the output tolerances.  Cases cover both tile forms (more and at most 64 query rows), FP16 KV,
partial last chunks, queries past the end of the cache and chunks that no query sees."""
import numpy as np
import pytest
import torch

import chunked_flashattention_q8_amd as q8a
from gpu_util import D, assert_close, dev, new_state, prefill, say
from test_gpu_attn import chunk_list, setup_case

pytestmark = pytest.mark.gpu

Q8, F16 = q8a.KV_Q8_0, q8a.KV_F16

CASES = [
    # B, H, M, N, q_pos0, chunk, kv dtype; the chunks cover keys [0, N) (N a multiple of 4)
    (1, 2, 200, 200, 0, 64, Q8),      # every row completed in its diagonal chunk, ragged tiles
    (2, 3, 132, 336, 204, 100, Q8),   # rows completed by the last two chunks, partial last chunk
    (1, 2, 31, 96, 65, 12, Q8),       # at most 64 rows (split-key form), many small chunks
    (2, 2, 33, 292, 259, 64, Q8),     # split-key form, the second block holds one row
    (1, 2, 300, 600, 100, 128, Q8),   # chunks past the last query position touch no row
    (1, 2, 100, 60, 0, 32, Q8),       # rows at positions 60..99 are never completed
    (2, 2, 200, 200, 0, 64, F16),     # FP16 KV
    (1, 3, 520, 520, 0, 520, Q8),     # one chunk completes every row
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_final_rows_match_finalize(orc, case, rows_per_workgroup):
    B, H, M, N, q_pos0, bc, kv = case
    say("case", case, "rows per workgroup", rows_per_workgroup)
    prob, qd, kd, vd = setup_case(orc, B, H, M, N, q_pos0, seed=sum(case[:6]), kv_dtype=kv)
    chunks = chunk_list(N, bc)
    out_ref, lse_ref, (m1, l1, o1) = prefill(qd, kd, vd, kv, B, H, M, N, q_pos0, chunks)

    row = q8a.ROW_BYTES[kv]
    st, (m, l, o) = new_state(B, H, M, q_pos0)
    # sentinels: the rows no chunk completes must keep them
    out = torch.full((B, H, M, D), 7.0, dtype=torch.float16, device=dev())
    lse = torch.full((B, H, M), -3.0, dtype=torch.float32, device=dev())
    kp, vp = kd.data_ptr(), vd.data_ptr()
    for s, n in chunks:
        q8a.attn_accumulate_chunk_final(st, qd, kp + s * row, vp + s * row, kv, s, n, N * row,
                                        H * N * row, out, lse)
    torch.cuda.synchronize()

    # the state: as the plain chunk calls left it (O of rows that stayed empty is never written)
    mg, lg = m.cpu().numpy().reshape(-1), l.cpu().numpy().reshape(-1)
    assert np.array_equal(mg.view(np.uint32), m1.cpu().numpy().reshape(-1).view(np.uint32))
    assert np.array_equal(lg.view(np.uint32), l1.cpu().numpy().reshape(-1).view(np.uint32))
    ne = ~np.isneginf(mg)
    assert np.array_equal(o.cpu().numpy().reshape(-1, D)[ne].view(np.uint32),
                          o1.cpu().numpy().reshape(-1, D)[ne].view(np.uint32))

    pos = q_pos0 + np.arange(M)
    done = np.tile(pos < N, B * H)  # completed by the chunk holding its position
    og = out.cpu().numpy().reshape(-1, D)
    lg2 = lse.cpu().numpy().reshape(-1)
    orf = out_ref.cpu().numpy().reshape(-1, D)
    lrf = lse_ref.cpu().numpy().reshape(-1)
    assert np.array_equal(og[done].view(np.uint16), orf[done].view(np.uint16))
    assert np.array_equal(lg2[done].view(np.uint32), lrf[done].view(np.uint32))
    assert np.all(og[~done] == np.float16(7.0)) and np.all(lg2[~done] == np.float32(-3.0))

    O_ref, lse_o = orc.attention(prob)
    if done.any():
        assert_close(og[done].astype(np.float32), lg2[done], O_ref[done], lse_o[done],
                     "completed rows " + str(case))


def test_final_without_lse(orc):
    """lse may be NULL: out alone is written, the same as with it."""
    B, H, M, N, q_pos0, bc = 1, 2, 130, 260, 0, 100
    prob, qd, kd, vd = setup_case(orc, B, H, M, N, q_pos0, seed=321)
    out_ref, _, _ = prefill(qd, kd, vd, Q8, B, H, M, N, q_pos0, chunk_list(N, bc))
    m, l, o = q8a.alloc_state(B, H, M)
    st = q8a.attn_state_init(m, l, o, B, H, M, D, q_pos0)
    out = torch.zeros((B, H, M, D), dtype=torch.float16, device=dev())
    for s, n in chunk_list(N, bc):
        q8a.attn_accumulate_chunk_final(st, qd, kd.data_ptr() + s * 68, vd.data_ptr() + s * 68,
                                        Q8, s, n, N * 68, H * N * 68, out, None)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_ref.view(torch.int16))


# ---------------------------------------------------------------- deferred initialisation and
# completed rows without their state (the flags of q8a_state)

DEFERRED = [
    # B, H, M, N, q_pos0, chunk, first chunk of the call order (the rest ascending)
    (1, 2, 200, 200, 0, 64, 0),      # every row sees the first chunk: no initialisation launch
    (2, 3, 130, 336, 203, 100, 0),   # q_pos0 past the first chunk's start
    (1, 2, 300, 640, 100, 128, 3),   # the first call's chunk (keys 384..511) starts after
                                     # q_pos0: the initialisation is enqueued before it
    (1, 2, 31, 96, 65, 12, 0),       # at most 64 rows (split-key form)
]


@pytest.mark.parametrize("case", DEFERRED, ids=[str(c) for c in DEFERRED])
def test_deferred_init_equals_init(orc, case, rows_per_workgroup):
    """attn_state_init_deferred then the chunk calls give the state, out and lse of
    attn_state_init then the same calls, bit for bit; the first call clears the FRESH bit."""
    B, H, M, N, q_pos0, bc, first = case
    say("deferred", case, "rows per workgroup", rows_per_workgroup)
    prob, qd, kd, vd = setup_case(orc, B, H, M, N, q_pos0, seed=sum(case))
    chunks = chunk_list(N, bc)
    chunks = chunks[first:first + 1] + chunks[:first] + chunks[first + 1:]
    out1, lse1, (m1, l1, o1) = prefill(qd, kd, vd, Q8, B, H, M, N, q_pos0, chunks)
    st, (m, l, o) = new_state(B, H, M, q_pos0, deferred=True)
    for t in (m, l, o):
        t.fill_(float("nan"))  # a deferred state's buffers may hold anything
    assert st.flags & q8a.STATE_FRESH
    kp, vp = kd.data_ptr(), vd.data_ptr()
    for i, (s, n) in enumerate(chunks):
        q8a.attn_accumulate_chunk(st, qd, kp + s * 68, vp + s * 68, Q8, s, n, N * 68,
                                  H * N * 68, 1)
        assert not st.flags & q8a.STATE_FRESH
    out = torch.empty_like(out1)
    lse = torch.empty_like(lse1)
    q8a.attn_finalize(st, out, lse)
    torch.cuda.synchronize()
    mm = m1.cpu().numpy().reshape(-1)
    assert np.array_equal(m.cpu().numpy().reshape(-1).view(np.uint32), mm.view(np.uint32))
    assert np.array_equal(l.cpu().numpy().reshape(-1).view(np.uint32),
                          l1.cpu().numpy().reshape(-1).view(np.uint32))
    ne = ~np.isneginf(mm)
    assert np.array_equal(o.cpu().numpy().reshape(-1, D)[ne].view(np.uint32),
                          o1.cpu().numpy().reshape(-1, D)[ne].view(np.uint32))
    assert torch.equal(out.view(torch.int16), out1.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse1.view(torch.int32))


@pytest.mark.parametrize("deferred", [False, True])
@pytest.mark.parametrize("case", [(1, 2, 200, 200, 0, 64, Q8), (2, 3, 132, 336, 204, 100, Q8),
                                  (1, 2, 31, 96, 65, 12, Q8), (2, 2, 200, 200, 0, 64, F16),
                                  (1, 3, 520, 520, 0, 520, Q8)])
def test_final_out_only(orc, case, deferred, rows_per_workgroup):
    """Q8A_STATE_FINAL_OUT_ONLY: the same out and lse bit for bit as the default chunk_final
    pass; the rows a call completes keep the state they held before that call, all other rows
    end as in the default pass.  With a deferred state too (the bench's step)."""
    B, H, M, N, q_pos0, bc, kv = case
    say("final out only", case, "deferred", deferred, "rows per workgroup", rows_per_workgroup)
    prob, qd, kd, vd = setup_case(orc, B, H, M, N, q_pos0, seed=sum(case[:6]), kv_dtype=kv)
    chunks = chunk_list(N, bc)
    row = q8a.ROW_BYTES[kv]
    kp, vp = kd.data_ptr(), vd.data_ptr()

    def run_pass(flags, snapshots):
        st, (m, l, o) = new_state(B, H, M, q_pos0, deferred=deferred, flags=flags)
        for t in (m, l, o):
            t.fill_(float("nan"))
        if not deferred:
            st = q8a.set_flags(q8a.attn_state_init(m, l, o, B, H, M, D, q_pos0), st.flags)
        out = torch.full((B, H, M, D), 7.0, dtype=torch.float16, device=dev())
        lse = torch.full((B, H, M), -3.0, dtype=torch.float32, device=dev())
        for s, n in chunks:
            if snapshots is not None:
                torch.cuda.synchronize()
                snapshots.append([t.cpu().numpy().copy() for t in (m, l, o)])
            q8a.attn_accumulate_chunk_final(st, qd, kp + s * row, vp + s * row, kv, s, n,
                                            N * row, H * N * row, out, lse)
        torch.cuda.synchronize()
        return out, lse, [t.cpu().numpy() for t in (m, l, o)]

    snaps = []
    out1, lse1, (m1, l1, o1) = run_pass(0, snaps)
    out2, lse2, (m2, l2, o2) = run_pass(q8a.STATE_FINAL_OUT_ONLY, None)
    assert torch.equal(out2.view(torch.int16), out1.view(torch.int16))
    assert torch.equal(lse2.view(torch.int32), lse1.view(torch.int32))
    pos = q_pos0 + np.arange(M)
    for ci, (s, n) in enumerate(chunks):
        done = (pos >= s) & (pos < s + n)  # rows this call completes keep their prior state
        sm, sl, so = snaps[ci]
        for got, want in ((m2, sm), (l2, sl)):
            np.testing.assert_array_equal(got[..., done].view(np.uint32),
                                          want[..., done].view(np.uint32))
        seen = ~np.isneginf(sm[..., done]) & ~np.isnan(sm[..., done])
        np.testing.assert_array_equal(o2[..., done, :][seen].view(np.uint32),
                                      so[..., done, :][seen].view(np.uint32))
    never = pos >= N  # rows no chunk completes: as in the default pass
    np.testing.assert_array_equal(m2[..., never].view(np.uint32), m1[..., never].view(np.uint32))
    np.testing.assert_array_equal(l2[..., never].view(np.uint32), l1[..., never].view(np.uint32))


def test_fresh_finalize_and_merge(orc):
    """A deferred state read before any chunk: finalize writes out = 0 and lse = -inf (the state
    is initialised first); merging it into a state leaves that state as it was; merging a
    state into it gives that state."""
    B, H, M, N, q_pos0 = 1, 2, 100, 100, 0
    prob, qd, kd, vd = setup_case(orc, B, H, M, N, q_pos0, seed=44)
    st, (m, l, o) = new_state(B, H, M, q_pos0, deferred=True)
    m.fill_(float("nan"))
    out = torch.full((B, H, M, D), 7.0, dtype=torch.float16, device=dev())
    lse = torch.zeros((B, H, M), dtype=torch.float32, device=dev())
    q8a.attn_finalize(st, out, lse)
    torch.cuda.synchronize()
    assert not st.flags & q8a.STATE_FRESH
    assert not out.any() and torch.all(torch.isneginf(lse))

    src, (mf, lf, of) = new_state(B, H, M, q_pos0)
    prefill(qd, kd, vd, Q8, B, H, M, N, q_pos0, chunk_list(N, 48), state=(src, (mf, lf, of)),
            finalize=False)
    fresh, (m2, l2, o2) = new_state(B, H, M, q_pos0, deferred=True)
    before = [t.clone() for t in (mf, lf, of)]
    q8a.attn_state_merge(src, fresh)       # FRESH src: nothing to merge
    torch.cuda.synchronize()
    assert fresh.flags & q8a.STATE_FRESH
    for a, b in zip(before, (mf, lf, of)):
        assert torch.equal(a, b)
    m2.fill_(float("nan"))
    q8a.attn_state_merge(fresh, src)       # FRESH dst takes src
    torch.cuda.synchronize()
    assert not fresh.flags & q8a.STATE_FRESH
    assert torch.equal(m2, mf) and torch.equal(l2, lf) and torch.equal(o2, of)
