"""Double-buffered host-to-device streaming ("Out-of-Core Flash Streaming & Speculative Decode
(1M Context)", Sec. 2: two ping-pong slots, chunk c+1 copied while chunk c is computed):
attn_accumulate_stream must give bit-for-bit the result of the same chunks fed from device
memory, and the 1M-token workload must match the oracle on its sampled rows."""
import numpy as np
import pytest
import torch

import chunked_flashattention_q8_amd as q8a
import synthetic
from gpu_util import D, assert_close, f16_to_dev, gpu_pack, prefill, rows_of, say

pytestmark = pytest.mark.gpu


def chunk_major(kd: torch.Tensor, chunk: int) -> torch.Tensor:
    """[1, H, N, 68] device bytes -> pinned host [C, 1, H, chunk, 68] (last chunk padded)."""
    _, H, N, R = kd.shape
    C = -(-N // chunk)
    host = torch.zeros((C, 1, H, chunk, R), dtype=torch.uint8, pin_memory=True)
    kc = kd.cpu()
    for c in range(C):
        n = min(chunk, N - c * chunk)
        host[c, 0, :, :n] = kc[0, :, c * chunk:c * chunk + n]
    return host


def run_stream(st, qd, kh, vh, n_total, chunk, H, n_seq=1):
    chunk_bytes = n_seq * H * chunk * 68
    slots_k = [torch.empty(chunk_bytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    slots_v = [torch.empty(chunk_bytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    copy = torch.cuda.Stream()
    q8a.attn_accumulate_stream(st, qd, kh, vh, q8a.KV_Q8_0, n_total, chunk, slots_k, slots_v, 1,
                               torch.cuda.current_stream(), copy)
    return slots_k, slots_v


@pytest.mark.parametrize("chunk", [64, 100])
def test_streamed_equals_resident(orc, chunk):
    H, M, N, q_pos0 = 4, 256, 1000, 744
    say("stream small", chunk)
    q, k, v = synthetic.small_case(1, H, M, N, q_pos0, seed=chunk)
    qd = f16_to_dev(q)
    kd, vd = gpu_pack(k), gpu_pack(v)
    torch.cuda.synchronize()
    chunks = [(s, min(chunk, N - s)) for s in range(0, N, chunk)]
    out_r, lse_r, _ = prefill(qd, kd, vd, q8a.KV_Q8_0, 1, H, M, N, q_pos0, chunks)
    kh, vh = chunk_major(kd, chunk), chunk_major(vd, chunk)
    m, l, o = q8a.alloc_state(1, H, M)
    st = q8a.attn_state_init(m, l, o, 1, H, M, D, q_pos0)
    keep = run_stream(st, qd, kh, vh, N, chunk, H)
    out = torch.empty_like(out_r)
    lse = torch.empty_like(lse_r)
    q8a.attn_finalize(st, out, lse)
    torch.cuda.synchronize()
    del keep
    assert torch.equal(out, out_r) and torch.equal(lse, lse_r)
    prob = orc.Problem(q, orc.q8_0_pack(k), orc.q8_0_pack(v), orc.KV_Q8_0, q_pos0)
    O_ref, lse_ref = orc.attention(prob)
    assert_close(out.float().cpu().numpy().reshape(-1, D), lse.cpu().numpy().reshape(-1),
                 O_ref, lse_ref, "stream %d" % chunk)


@pytest.mark.timeout(900)
def test_workload_stream_1m(orc):
    """1,048,576 keys (32 heads, 4.56 GB of Q8_0 K+V in pinned host memory) streamed in 64
    chunks of 16,384 tokens; 2048 queries at the end; 32 sampled rows per head."""
    w = synthetic.WORKLOADS[4]
    H, N, chunk = w.H, w.N, w.chunk
    C = w.n_chunks
    kh = torch.empty((C, 1, H, chunk, 68), dtype=torch.uint8, pin_memory=True)
    vh = torch.empty(kh.shape, dtype=torch.uint8, pin_memory=True)
    k_orc = np.empty((1, H, N, 68), dtype=np.uint8)
    v_orc = np.empty((1, H, N, 68), dtype=np.uint8)
    for c in range(C):
        k, v = synthetic.gen_kv_chunk(w, c)
        kb, vb = orc.q8_0_pack(k), orc.q8_0_pack(v)
        kd, vd = gpu_pack(k), gpu_pack(v)
        torch.cuda.synchronize()
        kg, vg = kd.cpu(), vd.cpu()
        assert np.array_equal(kg.numpy(), kb) and np.array_equal(vg.numpy(), vb), c
        kh[c, 0].copy_(kg)
        vh[c, 0].copy_(vg)
        k_orc[0, :, c * chunk:(c + 1) * chunk] = kb
        v_orc[0, :, c * chunk:(c + 1) * chunk] = vb
        if c % 8 == 0:
            say("packed chunk", c, "of", C)
    q = synthetic.gen_q(w)
    qd = f16_to_dev(q)
    m, l, o = q8a.alloc_state(1, H, w.M)
    st = q8a.attn_state_init(m, l, o, 1, H, w.M, D, w.q_pos0)
    say("streaming", C, "chunks")
    keep = run_stream(st, qd, kh, vh, N, chunk, H)
    out = torch.empty((1, H, w.M, D), dtype=torch.float16, device="cuda")
    lse = torch.empty((1, H, w.M), dtype=torch.float32, device="cuda")
    q8a.attn_finalize(st, out, lse)
    torch.cuda.synchronize()
    del keep
    rows = synthetic.sample_rows(w)
    say("oracle on", rows.size, "rows")
    prob = orc.Problem(q, k_orc, v_orc, orc.KV_Q8_0, w.q_pos0)
    O_ref, lse_ref = orc.attention(prob, rows)
    assert_close(rows_of(out, rows, D), rows_of(lse, rows), O_ref, lse_ref, w.name)
