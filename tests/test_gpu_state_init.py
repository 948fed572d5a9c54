"""attn_state_init marks every state row empty: m = -inf and l = 0 for exactly the
n_seq * n_heads * n_q rows, whatever the arrays' alignment (4-byte aligned suffices) and
whether or not the row count is a multiple of four; nothing before or after them is written."""
import numpy as np
import pytest
import torch

import chunked_flashattention_q8_amd as q8a
from gpu_util import D, dev, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape,off_m,off_l", [
    ((1, 1, 1), 0, 0),
    ((1, 1, 3), 1, 0),
    ((2, 3, 128), 0, 0),      # 768 rows, a multiple of 4
    ((1, 5, 251), 0, 0),      # 1255 rows: a ragged last group of four
    ((1, 5, 251), 3, 2),      # neither array 16-byte aligned
    ((3, 7, 1000), 2, 2),     # same misalignment in both
    ((8, 32, 2048), 0, 0),    # the batch-8 prefill state
])
def test_state_init_writes_exactly_the_rows(shape, off_m, off_l):
    B, H, M = shape
    rows = B * H * M
    say("state init", shape, off_m, off_l)
    pad = 64
    mb = torch.full((rows + 2 * pad,), 5.0, dtype=torch.float32, device=dev())
    lb = torch.full((rows + 2 * pad,), 6.0, dtype=torch.float32, device=dev())
    o = torch.empty((rows, D), dtype=torch.float32, device=dev())
    m_ptr = mb.data_ptr() + 4 * (pad + off_m)
    l_ptr = lb.data_ptr() + 4 * (pad + off_l)
    q8a.attn_state_init(m_ptr, l_ptr, o, B, H, M, D, 0)
    torch.cuda.synchronize()
    m = mb.cpu().numpy()
    l = lb.cpu().numpy()
    s_m, s_l = pad + off_m, pad + off_l
    assert np.all(np.isneginf(m[s_m:s_m + rows]))
    assert np.all(l[s_l:s_l + rows].view(np.uint32) == 0)
    assert np.all(m[:s_m] == 5.0) and np.all(m[s_m + rows:] == 5.0)
    assert np.all(l[:s_l] == 6.0) and np.all(l[s_l + rows:] == 6.0)
