"""The whole prefill step (pack K and V, state init, chunk calls, finalize) captured into a HIP
graph and replayed: every replay, with eager work and synchronisation between replays, must give
the eager output bit for bit.  The calls allocate nothing and launch only kernels (no memset or
copy nodes), so they are capturable as they stand."""
import pytest
import torch

import chunked_flashattention_q8_amd as q8a
import synthetic
from gpu_util import D, dev, f16_to_dev, say

pytestmark = pytest.mark.gpu


def test_graph_replays_equal_eager():
    w = synthetic.WORKLOADS[0]
    say("graph capture of workload", w.name)
    q = f16_to_dev(synthetic.gen_q(w))
    k, v = synthetic.gen_kv(w)
    kx, vx = torch.from_numpy(k).to(dev()), torch.from_numpy(v).to(dev())
    kd = torch.empty((w.B, w.H, w.N, 68), dtype=torch.uint8, device=dev())
    vd = torch.empty_like(kd)
    m, l, o = q8a.alloc_state(w.B, w.H, w.M)
    out = torch.empty((w.B, w.H, w.M, D), dtype=torch.float16, device=dev())
    lse = torch.empty((w.B, w.H, w.M), dtype=torch.float32, device=dev())
    n_rows = w.B * w.H * w.N

    def step():
        q8a.q8_0_pack(kx, kd, n_rows, 64)
        q8a.q8_0_pack(vx, vd, n_rows, 64)
        st = q8a.attn_state_init(m, l, o, w.B, w.H, w.M, D, w.q_pos0)
        for s, n in w.chunks():
            q8a.attn_accumulate_chunk(st, q, kd.data_ptr() + s * 68, vd.data_ptr() + s * 68,
                                      q8a.KV_Q8_0, s, n, w.N * 68, w.H * w.N * 68, 1)
        q8a.attn_finalize(st, out, lse)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = (out.clone(), lse.clone(), kd.clone())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for i in range(4):
        out.fill_(float("nan"))
        lse.zero_()
        kd.zero_()
        m.fill_(123.0)  # state init inside the graph must reset it
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1]), i
        assert torch.equal(kd, ref[2]), i
        step()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]), i


def test_graph_replays_lean_step_equal_eager():
    """The benchmark's step form captured: K and V packed side by side in one call, a deferred
    state (no init launch; the first chunk call initialises every row) with final-output-only
    rows, and the fused chunk calls that write each completed row's out and lse."""
    w = synthetic.WORKLOADS[0]
    say("graph capture of the lean step of workload", w.name)
    q = f16_to_dev(synthetic.gen_q(w))
    k, v = synthetic.gen_kv(w)
    kvx = torch.from_numpy(k).to(dev()).reshape(w.B, w.H, w.N, D)
    kvx = torch.stack([kvx, torch.from_numpy(v).to(dev()).reshape(w.B, w.H, w.N, D)])
    kvd = torch.empty((2, w.B, w.H, w.N, 68), dtype=torch.uint8, device=dev())
    m, l, o = q8a.alloc_state(w.B, w.H, w.M)
    out = torch.empty((w.B, w.H, w.M, D), dtype=torch.float16, device=dev())
    lse = torch.empty((w.B, w.H, w.M), dtype=torch.float32, device=dev())
    n_rows = w.B * w.H * w.N
    kp, vp = kvd[0].data_ptr(), kvd[1].data_ptr()

    def step():
        q8a.q8_0_pack(kvx, kvd, 2 * n_rows, 64)
        st = q8a.attn_state_init_deferred(m, l, o, w.B, w.H, w.M, D, w.q_pos0,
                                          q8a.STATE_FINAL_OUT_ONLY)
        for s, n in w.chunks():
            q8a.attn_accumulate_chunk_final(st, q, kp + s * 68, vp + s * 68, q8a.KV_Q8_0, s, n,
                                            w.N * 68, w.H * w.N * 68, out, lse)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = (out.clone(), lse.clone(), kvd.clone())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for i in range(4):
        out.fill_(float("nan"))
        lse.zero_()
        kvd.zero_()
        for t in (m, l, o):
            t.fill_(123.0)  # the deferred state must not read what a previous step left
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1]), i
        assert torch.equal(kvd, ref[2]), i
        step()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1]), i
