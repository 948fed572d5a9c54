"""Bytes after a chunk's last key never reach the result.  K and V buffers whose bytes after the
chunk are all 0xFF (a NaN in every FP16 position, Q8_0 scales included) give the same state, bit
for bit, as buffers holding zeros there.  Chunk lengths cover both unpack forms: byte lengths
that end on a 16-byte boundary (n_kv a multiple of 4 for Q8_0: nothing past the end is read)
and those that do not (the last 16-byte piece reads up to 12 bytes past the end, and the keys
they belong to are masked), in one- and two-tile chunks, causal and not."""
import numpy as np
import pytest
import torch

import chunked_flashattention_q8_amd as q8a
from gpu_util import D, dev, say
from test_gpu_attn import setup_case

pytestmark = pytest.mark.gpu


def run_chunk(qd, kbuf, vbuf, kv, B, H, M, n_kv, n_alloc, causal):
    row = q8a.ROW_BYTES[kv]
    m, l, o = q8a.alloc_state(B, H, M)
    st = q8a.attn_state_init(m, l, o, B, H, M, D, 0)
    q8a.attn_accumulate_chunk(st, qd, kbuf.data_ptr(), vbuf.data_ptr(), kv, 0, n_kv,
                              n_alloc * row, H * n_alloc * row, causal)
    torch.cuda.synchronize()
    mm = m.cpu().numpy().reshape(-1)
    ne = ~np.isneginf(mm)
    return (mm.view(np.uint32), l.cpu().numpy().reshape(-1).view(np.uint32),
            o.cpu().numpy().reshape(-1, D)[ne].view(np.uint32), o.cpu().numpy().reshape(-1, D)[ne])


@pytest.mark.parametrize("kv", [q8a.KV_Q8_0, q8a.KV_F16], ids=["q8_0", "f16"])
@pytest.mark.parametrize("n_kv", [1, 3, 4, 33, 60, 64, 65, 100, 128])
@pytest.mark.parametrize("causal", [1, 0])
def test_bytes_after_the_chunk_are_ignored(orc, kv, n_kv, causal):
    B, H, M = 1, 2, 130
    n_alloc = n_kv + 4 - n_kv % 4 + 8   # a multiple of 4 keys: 16-byte head strides
    say("chunk end", kv, n_kv, causal)
    _, qd, kd, vd = setup_case(orc, B, H, M, n_alloc, 0, seed=700 + n_kv, kv_dtype=kv)
    row = q8a.ROW_BYTES[kv]
    kb = kd.view(torch.uint8).reshape(B, H, n_alloc * row)
    vb = vd.view(torch.uint8).reshape(B, H, n_alloc * row)
    res = []
    for fill in (0x00, 0xFF):
        k2, v2 = kb.clone(), vb.clone()
        k2[:, :, n_kv * row:] = fill
        v2[:, :, n_kv * row:] = fill
        res.append(run_chunk(qd, k2, v2, kv, B, H, M, n_kv, n_alloc, causal))
    for a, b in zip(res[0][:3], res[1][:3]):
        assert np.array_equal(a, b)
    assert np.all(np.isfinite(res[1][3]))
