"""The layered workload (the pages' 16-layer model, "Out-of-Core Flash Streaming & Speculative
Decode (1M Context)", Sec. 1): every layer has its own Q, Q8_0 K/V cache (all resident in HBM)
and state, and a step runs the layers in turn.  Checked here at a reduced size with the code the
benchmark times (bench.run_layers): every layer's output against the oracle on all rows, and the
layers' outputs distinct (no state carried from one layer into the next)."""
import numpy as np
import pytest
import torch

import bench
import synthetic
from gpu_util import D, assert_close, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("chunk", [1024, 1000])
def test_layers_stream_each_against_oracle(orc, chunk):
    # 3 layers, 4 heads, 256 queries at the end of a 4096-token cache; chunk 1000 leaves a
    # partial last chunk
    w = synthetic.Workload(96, "layers_small", 1, 4, 256, 4096, 3840, chunk, None,
                           streamed=True, layers=3)
    say("layers", w.layers, "chunk", chunk)
    res = bench.run_layers(w, steps=1, warmup=1)
    torch.cuda.synchronize()
    outs = []
    for layer in range(w.layers):
        kb = np.empty((1, w.H, w.N, 68), dtype=np.uint8)
        vb = np.empty_like(kb)
        for c, (s0, n) in enumerate(w.chunks()):
            k, v = synthetic.gen_kv_chunk(w, c, layer)
            kb[0, :, s0:s0 + n] = orc.q8_0_pack(k)
            vb[0, :, s0:s0 + n] = orc.q8_0_pack(v)
        prob = orc.Problem(synthetic.gen_q(w, layer), kb, vb, orc.KV_Q8_0, w.q_pos0)
        O_ref, lse_ref = orc.attention(prob)
        out = res["outs"][layer].float().cpu().numpy().reshape(-1, D)
        lse = res["lses"][layer].cpu().numpy().reshape(-1)
        assert_close(out, lse, O_ref, lse_ref, "layer %d" % layer)
        outs.append(out)
    for a in range(w.layers):
        for b in range(a + 1, w.layers):
            assert not np.array_equal(outs[a], outs[b])
