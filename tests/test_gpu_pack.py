"""GPU q8_0_pack is bit-exact with the oracle's Q8_0 codec ("Core Architecture & The 4-Brick
Pipeline", Sec. 5, block_q8_0)."""
import numpy as np
import pytest
import torch

import chunked_flashattention_q8_amd as q8a
import synthetic
from gpu_util import dev, gpu_pack, say

pytestmark = pytest.mark.gpu


def pack_rows(x: np.ndarray, row_len: int) -> np.ndarray:
    xt = torch.from_numpy(np.ascontiguousarray(x)).to(dev())
    n_rows = x.size // row_len
    out = torch.empty(n_rows * row_len // 32 * 34, dtype=torch.uint8, device=dev())
    q8a.q8_0_pack(xt, out, n_rows, row_len)
    torch.cuda.synchronize()
    return out.cpu().numpy().reshape(x.shape[:-1] + (row_len // 32 * 34,))


@pytest.mark.parametrize("n_rows,row_len", [(1, 32), (3, 64), (1001, 64), (257, 96), (40000, 64)])
def test_pack_random_bitexact(orc, n_rows, row_len):
    rng = np.random.default_rng(n_rows)
    x = rng.standard_normal((n_rows, row_len)).astype(np.float32)
    x *= np.exp2(rng.uniform(-6, 9, size=(n_rows, 1))).astype(np.float32)
    say("pack", n_rows, row_len)
    assert np.array_equal(pack_rows(x, row_len), orc.q8_0_pack(x))


def test_pack_ties_zero_blocks_and_exact_scales(orc):
    rng = np.random.default_rng(5)
    blocks = []
    for s in (1.0, 0.5, 0.0078735352, 3.0, 2.0 ** -9):
        s = float(np.float16(s))
        k = rng.integers(-126, 126, size=(64, 32)) + 0.5 * (rng.random((64, 32)) < 0.5)
        k[:, 0] = 127
        blocks.append((k * s).astype(np.float32))
    # values one and two ulps either side of the exact ties: the quotient lands next to a
    # half-integer, where a product with the reciprocal of the scale may round differently
    for s in (1.0, 0.0078735352, 3.0):
        s = float(np.float16(s))
        k = (rng.integers(-126, 126, size=(64, 32)) + 0.5).astype(np.float32) * np.float32(s)
        for steps in (1, 2):
            away = np.where(rng.random(k.shape) < 0.5, np.float32(np.inf), np.float32(-np.inf))
            x = k.copy()
            for _ in range(steps):
                x = np.nextafter(x, away)
            x[:, 0] = np.float32(127 * s)
            blocks.append(x.astype(np.float32))
    blocks.append(np.zeros((8, 32), dtype=np.float32))
    tiny = rng.standard_normal((16, 32)).astype(np.float32) * np.float32(1e-3)  # subnormal d16
    blocks.append(tiny)
    x = np.concatenate(blocks).reshape(-1, 64)
    say("pack special blocks", x.shape)
    assert np.array_equal(pack_rows(x, 64), orc.q8_0_pack(x))


@pytest.mark.parametrize("wid", [0, 1, 2])
def test_pack_workload_kv(orc, wid):
    w = synthetic.WORKLOADS[wid]
    k, v = synthetic.gen_kv(w)
    for name, x in (("K", k), ("V", v)):
        say("pack workload", wid, name, x.shape)
        got = gpu_pack(x)
        torch.cuda.synchronize()
        assert np.array_equal(got.cpu().numpy(), orc.q8_0_pack(x)), name


@pytest.mark.parametrize("n_rows,row_len,offset", [(3, 32, 2), (1001, 32, 2), (777, 96, 2),
                                                   (777, 96, 4), (130, 32, 0)])
def test_pack_destination_alignment_and_odd_block_counts(orc, n_rows, row_len, offset):
    """dst only 2-byte aligned (offset 2) and odd block counts (the last 2-byte piece of a
    workgroup's range); the bytes around the packed range are left untouched."""
    rng = np.random.default_rng(n_rows + offset)
    x = rng.standard_normal((n_rows, row_len)).astype(np.float32)
    xt = torch.from_numpy(x).to(dev())
    n_bytes = n_rows * row_len // 32 * 34
    buf = torch.full((n_bytes + 16,), 0xA5, dtype=torch.uint8, device=dev())
    say("pack to offset", offset, n_rows, row_len)
    q8a.q8_0_pack(xt, buf.data_ptr() + offset, n_rows, row_len)
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    assert np.array_equal(got[offset:offset + n_bytes], orc.q8_0_pack(x).reshape(-1))
    assert (got[:offset] == 0xA5).all() and (got[offset + n_bytes:] == 0xA5).all()


def test_pack_scales_across_the_fp16_range(orc):
    """Block maxima from 1e-9 to 3e4 (FP16 scales that are zero, subnormal, normal and near the
    largest finite value), a dense sweep of maxima around 127 * 2^-14 (where the FP16 scale turns
    from subnormal to normal), then the same blocks with most values moved onto the
    quantiser's ties of their own scale and 0, 1 or 2 ulps either side."""
    rng = np.random.default_rng(11)
    amax = np.exp(rng.uniform(np.log(1e-9), np.log(3e4), size=4096))
    sweep = 127 * 2.0 ** -14 * (1 + np.linspace(-0.02, 0.02, 2048))
    amax = np.concatenate([amax, sweep]).astype(np.float32)
    x = (rng.uniform(-1, 1, size=(amax.size, 32)) * amax[:, None]).astype(np.float32)
    x[:, 0] = amax
    say("pack scale range", x.shape)
    ref = orc.q8_0_pack(x.reshape(-1, 64))
    assert np.array_equal(pack_rows(x.reshape(-1, 64), 64), ref)
    d16 = ref.reshape(-1, 34)[:, :2].copy().view(np.float16).astype(np.float32).reshape(-1)
    k = rng.integers(-126, 126, size=(amax.size, 31)) + 0.5
    t = (k * d16[:, None]).astype(np.float32)
    for _ in range(2):
        step = rng.integers(-1, 2, size=t.shape)
        t = np.where(step > 0, np.nextafter(t, np.float32(np.inf)),
                     np.where(step < 0, np.nextafter(t, np.float32(-np.inf)), t)).astype(np.float32)
    x[:, 1:] = t
    say("pack scale range, ties", x.shape)
    assert np.array_equal(pack_rows(x.reshape(-1, 64), 64), orc.q8_0_pack(x.reshape(-1, 64)))
