"""The benchmark's own step at the workloads' full sizes, against the oracle: K and V packed
side by side by one q8_0_pack call, the state described by attn_state_init_deferred with
Q8A_STATE_FINAL_OUT_ONLY (no init launch), and the chunk calls of attn_accumulate_chunk_final
writing the final out/lse of the rows each completes ("Out-of-Core Flash Streaming & Speculative
Decode (1M Context)", Sec. 3: the recurrence over chunks, the final normalisation as soon as a
row has seen its last key) -- the launch configuration bench.py times.  The step runs twice on
the same buffers, as the timed steps do; the packed bytes are checked bit for bit and out/lse on
the oracle's sampled rows."""
import numpy as np
import pytest
import torch

import chunked_flashattention_q8_amd as q8a
import synthetic
from gpu_util import D, assert_close, dev, rows_of, say

pytestmark = pytest.mark.gpu


def lean_step(w, qd, kvx, kvd, chunk, out, lse, m, l, o):
    n_rows = w.B * w.H * w.N
    q8a.q8_0_pack(kvx, kvd, 2 * n_rows, 64)
    st = q8a.attn_state_init_deferred(m, l, o, w.B, w.H, w.M, D, w.q_pos0,
                                      q8a.STATE_FINAL_OUT_ONLY)
    kp, vp = kvd[0].data_ptr(), kvd[1].data_ptr()
    for s in range(0, w.N, chunk):
        n = min(chunk, w.N - s)
        q8a.attn_accumulate_chunk_final(st, qd, kp + s * 68, vp + s * 68, q8a.KV_Q8_0, s, n,
                                        w.N * 68, w.H * w.N * 68, out, lse)
    assert not (st.flags & q8a.STATE_FRESH)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("wid", [1, 2])
def test_bench_step_full_size(orc, wid):
    w = synthetic.WORKLOADS[wid]
    say("bench step", w.name, "B_C", w.chunk)
    q = synthetic.gen_q(w)
    k, v = synthetic.gen_kv(w)
    qd = torch.from_numpy(q).view(torch.float16).to(dev())
    kvx = torch.empty((2, w.B, w.H, w.N, D), dtype=torch.float32, device=dev())
    kvx[0].copy_(torch.from_numpy(k))
    kvx[1].copy_(torch.from_numpy(v))
    kvd = torch.empty((2, w.B, w.H, w.N, 68), dtype=torch.uint8, device=dev())
    m, l, o = q8a.alloc_state(w.B, w.H, w.M, dev())
    out = torch.empty((w.B, w.H, w.M, D), dtype=torch.float16, device=dev())
    lse = torch.empty((w.B, w.H, w.M), dtype=torch.float32, device=dev())
    lean_step(w, qd, kvx, kvd, w.chunk, out, lse, m, l, o)
    torch.cuda.synchronize()
    first = (out.clone(), lse.clone())
    lean_step(w, qd, kvx, kvd, w.chunk, out, lse, m, l, o)
    torch.cuda.synchronize()
    assert torch.equal(out, first[0]) and torch.equal(lse, first[1])
    kb, vb = orc.q8_0_pack(k), orc.q8_0_pack(v)
    assert np.array_equal(kvd[0].cpu().numpy(), kb)
    assert np.array_equal(kvd[1].cpu().numpy(), vb)
    del kvx, k, v
    rows = synthetic.sample_rows(w, 16)
    prob = orc.Problem(q, kb, vb, orc.KV_Q8_0, w.q_pos0)
    O_ref, lse_ref = orc.attention(prob, rows)
    assert_close(rows_of(out, rows, D), rows_of(lse, rows), O_ref, lse_ref,
                 w.name + " bench step")
