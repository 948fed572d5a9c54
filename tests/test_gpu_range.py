"""The edges of the supported value range (finite K and V with |x| < 30000) on the attention
path, against the FP64 oracle.  Large Q8_0 scales reach the unpack's FP16 intermediates (the V
values fp16(q * d) up to 29000; the K scale factors d0 / d1 and d1 * log2(e) / 8) and FP32 logits
of the same size; a test with N(0, 1) data never does.

* large V: V of a few thousand (clipped to +-29000), Q and K N(0, 1).  The FP16 output grid is
  then 2 to 16 apart, so the absolute max-abs bound of 2e-3 would measure the output format; it
  is applied per unit of the V scale instead (2e-3 x 6000), while rel-RMS (1e-3) and LSE
  (1e-4) keep their bounds.
* large K: K of a few thousand (clipped to +-29000) and Q divided by the same scale, so the
  logits stay about N(0, 1) while every K block scale is large; all bounds as stated.
* mixed: every Q8_0 block of every key scaled by its own factor spread over six decades (0.01 to
  20000), Q divided by 100: the softmax is dominated by a few keys, and the ratios d0 / d1 of a
  key's two block scales span about twelve decades.  V is N(0, 0.5^2), as in the rescale tests:
  a row dominated by one key has |O| near that key's |V|, and at |O| in [2, 4) the FP16 output
  grid and the FP16 weights alone put about 1e-3 of error on each such value.

Each case runs under every tile form and the at most 64-row split form."""
import numpy as np
import pytest
import torch

import chunked_flashattention_q8_amd as q8a
import synthetic
from gpu_util import D, assert_close, f16_to_dev, gpu_pack, metrics, prefill, say
from test_gpu_attn import chunk_list

pytestmark = pytest.mark.gpu

SCALE = 6000.0
CASES = [(1, 2, 200, 332, 132, 64), (1, 2, 48, 400, 352, 100)]  # B, H, M, N, q_pos0, chunk


def _draw(kind, B, H, M, N, q_pos0, seed):
    q, k, v = synthetic.small_case(B, H, M, N, q_pos0, seed)
    rng = np.random.default_rng(seed)
    if kind == "large_v":
        v = np.clip(v * SCALE, -29000, 29000).astype(np.float32)
    elif kind == "large_k":
        k = np.clip(k * SCALE, -29000, 29000).astype(np.float32)
        q = synthetic.to_f16_bits(q.view(np.float16).astype(np.float32) / np.float32(SCALE))
    else:  # mixed: each block of each key scaled by its own 10^u, u uniform in [-2, 4.3]
        s = np.power(10.0, rng.uniform(-2.0, 4.3, size=(B, H, N, 2, 1))).astype(np.float32)
        k = np.clip(k.reshape(B, H, N, 2, 32) * s, -29000, 29000).reshape(B, H, N, D)
        k = k.astype(np.float32)
        q = synthetic.to_f16_bits(q.view(np.float16).astype(np.float32) / np.float32(100.0))
        v = (v * np.float32(0.5)).astype(np.float32)
    return q, k, v


@pytest.mark.parametrize("kind", ["large_v", "large_k", "mixed"])
@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_value_range(orc, kind, case, rows_per_workgroup):
    B, H, M, N, q_pos0, bc = case
    q, k, v = _draw(kind, B, H, M, N, q_pos0, seed=71)
    assert np.abs(k).max() < 30000 and np.abs(v).max() < 30000
    kd, vd = gpu_pack(k), gpu_pack(v)
    kb, vb = orc.q8_0_pack(k), orc.q8_0_pack(v)
    torch.cuda.synchronize()
    assert np.array_equal(kd.cpu().numpy(), kb) and np.array_equal(vd.cpu().numpy(), vb)
    prob = orc.Problem(q, kb, vb, orc.KV_Q8_0, q_pos0)
    say("value range", kind, case, rows_per_workgroup)
    out, lse, _ = prefill(f16_to_dev(q), kd, vd, q8a.KV_Q8_0, B, H, M, N, q_pos0,
                          chunk_list(N, bc))
    O_ref, lse_ref = orc.attention(prob)
    o = out.float().cpu().numpy().reshape(-1, D)
    l = lse.cpu().numpy().reshape(-1)
    assert np.isfinite(o).all() and np.isfinite(l).all()
    if kind == "large_v":
        max_abs, rel_rms, lse_err = metrics(o, l, O_ref, lse_ref)
        say("  max-abs %.3e (bound %.3e) rel-rms %.3e lse-rel %.3e" % (max_abs, 2e-3 * SCALE,
                                                                       rel_rms, lse_err))
        assert max_abs <= 2e-3 * SCALE and rel_rms <= 1e-3 and lse_err <= 1e-4
    else:
        assert_close(o, l, O_ref, lse_ref, kind)
