"""Seeded random cases against the FP64 oracle: shapes, query offsets, chunkings (ragged last
chunk, shuffled order), causal and not, Q8_0 and FP16 KV, every tile form, and the three ways of
running a pass -- plain chunk calls and a finalize launch, fused chunk calls that write the rows
each completes, and the deferred final-out-only state the benchmark step uses ("Out-of-Core
Flash Streaming & Speculative Decode (1M Context)", Sec. 3: the chunk recurrence; the result
equals single-pass attention whatever the chunking).  Each case is drawn from its own seed, so a
failure names a reproducible case."""
import numpy as np
import pytest
import torch

import chunked_flashattention_q8_amd as q8a
import gpu_util
import synthetic
from gpu_util import D, assert_close, dev, f16_to_dev, gpu_pack, say

pytestmark = pytest.mark.gpu

FORMS = ["auto", "128", "256", "256k", "64"]


def draw(seed):
    r = np.random.default_rng(1000 + seed)
    B, H = int(r.integers(1, 3)), int(r.integers(1, 4))
    M = int(r.choice([1, 7, 31, 32, 33, 64, 65, 100, 128, 129, 200, 256, 257, 320]))
    causal = int(r.random() < 0.75)
    kv = q8a.KV_Q8_0 if r.random() < 0.75 else q8a.KV_F16
    mode = str(r.choice(["plain", "fused", "lean"])) if causal else "plain"
    if causal:
        n_cover = int(r.integers(M, M + 600))
        q_pos0 = int(r.integers(0, n_cover - M + 1))
    else:
        n_cover = int(r.integers(1, 180)) * 4
        q_pos0 = int(r.integers(0, 2000))
    n_alloc = (n_cover + 3) // 4 * 4
    # chunks: lengths that are multiples of 4 keys (16-byte chunk starts), the last one ragged
    chunks, s = [], 0
    while s < n_cover:
        n = min(int(r.integers(1, 80)) * 4, n_cover - s)
        chunks.append((s, n))
        s += n
    if mode == "plain" and r.random() < 0.5:
        chunks = [chunks[i] for i in r.permutation(len(chunks))]
    form = str(r.choice(FORMS))
    return dict(B=B, H=H, M=M, n_cover=n_cover, n_alloc=n_alloc, q_pos0=q_pos0, causal=causal,
                kv=kv, mode=mode, chunks=chunks, form=form)


@pytest.mark.parametrize("seed", range(160))
def test_random_case(orc, seed):
    c = draw(seed)
    B, H, M, q_pos0, kv = c["B"], c["H"], c["M"], c["q_pos0"], c["kv"]
    say("seed", seed, {k: v for k, v in c.items() if k != "chunks"}, "chunks", len(c["chunks"]))
    q, k, v = synthetic.small_case(B, H, M, c["n_alloc"], q_pos0, seed=7000 + seed)
    qd = f16_to_dev(q)
    if kv == q8a.KV_Q8_0:
        kd, vd = gpu_pack(k), gpu_pack(v)
        kb, vb = orc.q8_0_pack(k), orc.q8_0_pack(v)
        prob = orc.Problem(q, kb, vb, orc.KV_Q8_0, q_pos0)
    else:
        kb, vb = synthetic.to_f16_bits(k), synthetic.to_f16_bits(v)
        kd, vd = f16_to_dev(kb), f16_to_dev(vb)
        prob = orc.Problem(q, kb, vb, orc.KV_F16, q_pos0)
    prob.causal = bool(c["causal"])
    row = q8a.ROW_BYTES[kv]
    N = c["n_alloc"]
    gpu_util.TILE_FORM[0] = gpu_util.FORMS[c["form"]]
    try:
        if c["mode"] == "lean":
            st, (m, l, o) = gpu_util.new_state(B, H, M, q_pos0, deferred=True,
                                                flags=q8a.STATE_FINAL_OUT_ONLY)
        else:
            st, (m, l, o) = gpu_util.new_state(B, H, M, q_pos0)
    finally:
        gpu_util.TILE_FORM[0] = gpu_util.FORMS["auto"]
    out = torch.full((B, H, M, D), float("nan"), dtype=torch.float16, device=dev())
    lse = torch.full((B, H, M), float("nan"), dtype=torch.float32, device=dev())
    kp, vp = kd.data_ptr(), vd.data_ptr()
    for s, n in c["chunks"]:
        if c["mode"] == "plain":
            q8a.attn_accumulate_chunk(st, qd, kp + s * row, vp + s * row, kv, s, n, N * row,
                                      H * N * row, c["causal"])
        else:
            q8a.attn_accumulate_chunk_final(st, qd, kp + s * row, vp + s * row, kv, s, n,
                                            N * row, H * N * row, out, lse)
    if c["mode"] == "plain":
        q8a.attn_finalize(st, out, lse)
    torch.cuda.synchronize()
    O_ref, lse_ref = orc.attention(prob)
    assert_close(out.float().cpu().numpy().reshape(-1, D), lse.cpu().numpy().reshape(-1),
                 O_ref, lse_ref, "seed %d" % seed)
