"""attn_accumulate_file (the out-of-core feed from storage of "Out-of-Core Flash Streaming &
Speculative Decode (1M Context)", Sec. 2: chunks read with the page cache bypassed into a
two-slot ring) on the GPU.  Files opened with O_DIRECT, a header before the cache so that no chunk
starts on a 4096-byte boundary, chunks whose size is not a multiple of 4096 and a partial last
chunk: the result equals the pinned-host stream's bit for bit and the oracle's within the bounds;
a file that ends early returns Q8A_E_IO with exactly the chunks before it accumulated."""
import os

import numpy as np
import pytest
import torch

import chunked_flashattention_q8_amd as q8a
import synthetic
from gpu_util import D, assert_close, dev, f16_to_dev, say

pytestmark = pytest.mark.gpu

B, H, M, N, Q_POS0, CHUNK, HEADER = 2, 3, 200, 777, 577, 256, 100


def chunk_major(packed, chunk):
    """[B, H, N, 68] -> [C, B, H, chunk, 68] (the last chunk zero-padded)."""
    b, h, n, r = packed.shape
    c = -(-n // chunk)
    out = np.zeros((c, b, h, chunk, r), dtype=np.uint8)
    for i in range(c):
        s = i * chunk
        e = min(n, s + chunk)
        out[i, :, :, :e - s] = packed[:, :, s:e]
    return out


def write_file(path, body, header=HEADER):
    with open(path, "wb") as f:
        f.write(bytes([0x5A]) * header)
        f.write(body.tobytes())


def run(st_buffers, qd, fn):
    m, l, o = st_buffers
    st = q8a.attn_state_init(m, l, o, B, H, M, D, Q_POS0)
    rc = fn(st)
    out = torch.empty((B, H, M, D), dtype=torch.float16, device=dev())
    lse = torch.empty((B, H, M), dtype=torch.float32, device=dev())
    q8a.attn_finalize(st, out, lse)
    torch.cuda.synchronize()
    return rc, out, lse


def setup(orc, tmp_path):
    q, k, v = synthetic.small_case(B, H, M, N, Q_POS0, seed=71)
    kb, vb = orc.q8_0_pack(k), orc.q8_0_pack(v)
    kc, vc = chunk_major(kb, CHUNK), chunk_major(vb, CHUNK)
    pk, pv = str(tmp_path / "k.q8"), str(tmp_path / "v.q8")
    write_file(pk, kc)
    write_file(pv, vc)
    return q, kb, vb, kc, vc, pk, pv


def open_direct(path):
    return os.open(path, os.O_RDONLY | getattr(os, "O_DIRECT", 0))


@pytest.mark.parametrize("direct", [True, False])
def test_file_feed_equals_host_stream_and_oracle(orc, tmp_path, direct):
    """O_DIRECT descriptors with an mmap'd ring, buffered descriptors with a pinned ring."""
    q, kb, vb, kc, vc, pk, pv = setup(orc, tmp_path)
    qd = f16_to_dev(q)
    cb = B * H * CHUNK * 68
    say("file feed, chunk bytes", cb, "header", HEADER, "O_DIRECT", direct)
    slots_k = [torch.empty(cb, dtype=torch.uint8, device=dev()) for _ in range(2)]
    slots_v = [torch.empty(cb, dtype=torch.uint8, device=dev()) for _ in range(2)]
    ring_k = q8a.alloc_ring(cb + 8192, pinned=not direct)
    ring_v = q8a.alloc_ring(cb + 8192, pinned=not direct)
    bufs = q8a.alloc_state(B, H, M)
    cs, ds = torch.cuda.current_stream(), torch.cuda.Stream()
    if direct:
        fk, fv = open_direct(pk), open_direct(pv)
    else:
        fk, fv = os.open(pk, os.O_RDONLY), os.open(pv, os.O_RDONLY)
    try:
        _, out_f, lse_f = run(bufs, qd, lambda st: q8a.attn_accumulate_file(
            st, qd, fk, fv, HEADER, q8a.KV_Q8_0, N, CHUNK, ring_k, ring_v, cb + 8192, slots_k,
            slots_v, 1, cs, ds))
    finally:
        os.close(fk)
        os.close(fv)
    state_f = [t.cpu() for t in bufs]
    kh = torch.from_numpy(kc.reshape(-1)).pin_memory()
    vh = torch.from_numpy(vc.reshape(-1)).pin_memory()
    _, out_s, lse_s = run(bufs, qd, lambda st: q8a.attn_accumulate_stream(
        st, qd, kh, vh, q8a.KV_Q8_0, N, CHUNK, slots_k, slots_v, 1, cs, ds))
    for a, b_ in zip(state_f, bufs):
        assert torch.equal(a, b_.cpu())
    assert torch.equal(out_f, out_s) and torch.equal(lse_f, lse_s)
    prob = orc.Problem(q, kb, vb, orc.KV_Q8_0, Q_POS0)
    O_ref, lse_ref = orc.attention(prob)
    assert_close(out_f.float().cpu().numpy().reshape(-1, D), lse_f.cpu().numpy().reshape(-1),
                 O_ref, lse_ref, "file feed")


def test_file_that_ends_early(orc, tmp_path):
    q, kb, vb, kc, vc, pk, pv = setup(orc, tmp_path)
    qd = f16_to_dev(q)
    cb = B * H * CHUNK * 68
    # the V file ends inside chunk 2: chunks 0 and 1 are accumulated, then Q8A_E_IO
    with open(pv, "r+b") as f:
        f.truncate(HEADER + 2 * cb + 1000)
    slots_k = [torch.empty(cb, dtype=torch.uint8, device=dev()) for _ in range(2)]
    slots_v = [torch.empty(cb, dtype=torch.uint8, device=dev()) for _ in range(2)]
    ring_k, ring_v = q8a.alloc_ring(cb + 8192), q8a.alloc_ring(cb + 8192)
    bufs = q8a.alloc_state(B, H, M)
    cs, ds = torch.cuda.current_stream(), torch.cuda.Stream()
    fk, fv = open_direct(pk), open_direct(pv)
    say("file ending inside chunk 2")

    def feed(st):
        try:
            q8a.attn_accumulate_file(st, qd, fk, fv, HEADER, q8a.KV_Q8_0, N, CHUNK, ring_k,
                                     ring_v, cb + 8192, slots_k, slots_v, 1, cs, ds)
        except q8a.Q8AError as e:
            return e.status
        return q8a.Q8A_OK
    try:
        rc, out_f, lse_f = run(bufs, qd, feed)
    finally:
        os.close(fk)
        os.close(fv)
    assert rc == q8a.Q8A_E_IO
    state_f = [t.cpu() for t in bufs]
    kh = torch.from_numpy(kc.reshape(-1)).pin_memory()
    vh = torch.from_numpy(vc.reshape(-1)).pin_memory()
    run(bufs, qd, lambda st: q8a.attn_accumulate_stream(
        st, qd, kh, vh, q8a.KV_Q8_0, 2 * CHUNK, CHUNK, slots_k, slots_v, 1, cs, ds))
    for a, b_ in zip(state_f, bufs):
        assert torch.equal(a, b_.cpu())
