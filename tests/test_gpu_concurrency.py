"""Calls on different states are independent.  Two problems, each with its own Q, K/V and state,
are accumulated chunk by chunk with their calls interleaved on two streams and no
synchronisation between the streams; each must give bit for bit what it gives alone on one
stream, and match the oracle.  One is a 256-row-form causal prefill through the fused
final-output calls on a deferred state; the other a 64-row split-form pass over FP16 keys and
values ending in a finalize launch, so the two streams run different kernels side by side."""
import pytest
import torch

import chunked_flashattention_q8_amd as q8a
import synthetic
from gpu_util import D, assert_close, dev, f16_to_dev, gpu_pack, say

pytestmark = pytest.mark.gpu


def _problem(orc, B, H, M, N, q_pos0, seed, kv_dtype, causal):
    q, k, v = synthetic.small_case(B, H, M, N, q_pos0, seed)
    if kv_dtype == q8a.KV_Q8_0:
        kb, vb = orc.q8_0_pack(k), orc.q8_0_pack(v)
        kd, vd = gpu_pack(k), gpu_pack(v)
        prob = orc.Problem(q, kb, vb, orc.KV_Q8_0, q_pos0, bool(causal))
    else:
        kb, vb = synthetic.to_f16_bits(k), synthetic.to_f16_bits(v)
        kd, vd = f16_to_dev(kb), f16_to_dev(vb)
        prob = orc.Problem(q, kb, vb, orc.KV_F16, q_pos0, bool(causal))
    return dict(causal=causal, B=B, H=H, M=M, N=N, q_pos0=q_pos0, kv=kv_dtype, prob=prob, q=f16_to_dev(q),
                k=kd, v=vd, row=q8a.ROW_BYTES[kv_dtype])


class _Run:
    """One problem's state and outputs; step(i) enqueues its i-th call on the current stream."""

    def __init__(self, p, chunk, fused):
        self.p, self.fused = p, fused
        B, H, M, N = p["B"], p["H"], p["M"], p["N"]
        self.m, self.l, self.o = q8a.alloc_state(B, H, M)
        self.out = torch.zeros((B, H, M, D), dtype=torch.float16, device=dev())
        self.lse = torch.zeros((B, H, M), dtype=torch.float32, device=dev())
        self.chunks = [(s, min(chunk, N - s)) for s in range(0, N, chunk)]
        if fused:
            self.st = q8a.attn_state_init_deferred(self.m, self.l, self.o, B, H, M, D,
                                                   p["q_pos0"], q8a.STATE_FINAL_OUT_ONLY)
        else:
            self.st = None

    def n_calls(self):
        return len(self.chunks) + (0 if self.fused else 2)  # + init and finalize

    def step(self, i):
        p = self.p
        hs, ss = p["N"] * p["row"], p["H"] * p["N"] * p["row"]
        if not self.fused:
            if i == 0:
                self.st = q8a.attn_state_init(self.m, self.l, self.o, p["B"], p["H"], p["M"], D,
                                              p["q_pos0"])
                return
            i -= 1
            if i == len(self.chunks):
                q8a.attn_finalize(self.st, self.out, self.lse)
                return
        s, n = self.chunks[i]
        kp, vp = p["k"].data_ptr() + s * p["row"], p["v"].data_ptr() + s * p["row"]
        if self.fused:
            q8a.attn_accumulate_chunk_final(self.st, p["q"], kp, vp, p["kv"], s, n, hs, ss,
                                            self.out, self.lse)
        else:
            q8a.attn_accumulate_chunk(self.st, p["q"], kp, vp, p["kv"], s, n, hs, ss, p["causal"])


def test_two_states_on_two_streams(orc):
    pa = _problem(orc, 2, 3, 300, 700, 400, seed=41, kv_dtype=q8a.KV_Q8_0, causal=1)
    pb = _problem(orc, 1, 4, 64, 900, 836, seed=42, kv_dtype=q8a.KV_F16, causal=0)
    torch.cuda.synchronize()

    def alone():
        ra, rb = _Run(pa, 128, True), _Run(pb, 100, False)
        for r in (ra, rb):
            for i in range(r.n_calls()):
                r.step(i)
        torch.cuda.synchronize()
        return ra, rb

    ref_a, ref_b = alone()
    for name, r, p in (("A", ref_a, pa), ("B", ref_b, pb)):
        O_ref, lse_ref = orc.attention(p["prob"])
        assert_close(r.out.float().cpu().numpy().reshape(-1, D), r.lse.cpu().numpy().reshape(-1),
                     O_ref, lse_ref, name + " alone")
    for rep in range(2):
        ra, rb = _Run(pa, 128, True), _Run(pb, 100, False)
        sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
        main = torch.cuda.current_stream()
        sa.wait_stream(main)
        sb.wait_stream(main)
        say("interleaved on two streams, pass", rep, ra.n_calls(), rb.n_calls())
        for i in range(max(ra.n_calls(), rb.n_calls())):
            if i < ra.n_calls():
                with torch.cuda.stream(sa):
                    ra.step(i)
            if i < rb.n_calls():
                with torch.cuda.stream(sb):
                    rb.step(i)
        main.wait_stream(sa)
        main.wait_stream(sb)
        torch.cuda.synchronize()
        assert torch.equal(ra.out, ref_a.out) and torch.equal(ra.lse, ref_a.lse)
        assert torch.equal(rb.out, ref_b.out) and torch.equal(rb.lse, ref_b.lse)
        assert torch.equal(rb.m, ref_b.m) and torch.equal(rb.l, ref_b.l) and torch.equal(rb.o, ref_b.o)
