"""Seeded synthetic workloads shared by the tests, the smoke check and the benchmark.

This module only draws inputs; it holds none of the method's arithmetic (no quantisation, no
attention).  Both the HIP path and the CPU oracle are fed from here, and nothing else is shared
between them.

Workloads (shapes of the pages' prefill workloads: head_dim 64, 32 heads, the M <= 2048 release
scope, a ~130K-token append and a 1M-token context; values N(0, 1)):

====  ==================  ==  ==  =====  =========  =========  =======  =========
id    name                B   H   M      N          q_pos0     B_C      checked
====  ==================  ==  ==  =====  =========  =========  =======  =========
0     tiny                1   4   256    256        0          64       all rows
1     incore_m2048        1   32  2048   2048       0          512      all rows
2     batch8_m2048        8   32  2048   2048       0          512      sampled
3     append_133k         1   32  2048   133120     131072     8192     64/head
4     stream_1m           1   32  2048   1048576    1046528    16384    32/head
5     burst_verify_1m     1   32  64     1048576    1048576    16384    all rows
6     layers16_1m       1   32  2048   1048576    1046528    16384    2/head, 2 layers
====  ==================  ==  ==  =====  =========  =========  =======  =========

Workload 5 is Mode B of "Out-of-Core Flash Streaming & Speculative Decode (1M Context)", Sec. 4:
64 candidate queries (positions just past the cache) attend to the whole 1M-token context with
no causal mask.  Workload 6 is workload 4 for each of 16 layers (the pages' 16-layer model: 16
caches of 4.56 GB), every layer with its own Q, K, V and state; it is drawn per chunk like the
streamed workloads and held resident in HBM.

Draws: every tensor is a stack of [rows, 64] slices, one per (sequence, head); slice i of a
tensor with seed s is filled by ``torch.Tensor.normal_`` (float32, mean 0, std 1) from its own
``torch.Generator`` seeded ``s * 1_000_003 + i``, so slices can be drawn on parallel threads and
the values do not depend on the thread count.  For workload k, Q uses seed ``1000*k + 1``, K
``1000*k + 2`` and V ``1000*k + 3``.  Q is then stored as FP16 (round to nearest even) because
the method's queries are FP16; K and V stay float32 (they are quantised by the method).  The
streamed 1M-token workload draws K and V per chunk c with seeds ``1000*k + 100 + 2c`` and
``1000*k + 101 + 2c`` and shape [H, B_C, 64], so no process ever holds the whole float32 cache.
Layer l of a layered workload adds ``100_000 * l`` to each of these seeds (layer 0 keeps them).
Sampled query rows come from ``numpy.random.default_rng(1000*k + 9)``, drawn per head without
replacement, always including rows 0 and M - 1.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np
import torch

HEAD_DIM = 64


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    B: int
    H: int
    M: int
    N: int
    q_pos0: int
    chunk: int
    rows_per_head: int | None  # None = every row is checked
    streamed: bool = False
    causal: bool = True
    layers: int = 1

    @property
    def D(self) -> int:
        return HEAD_DIM

    @property
    def n_chunks(self) -> int:
        return -(-self.N // self.chunk)

    def chunks(self):
        """[(kv_pos0, n_kv), ...] in ascending order; the last one may be partial."""
        return [(c * self.chunk, min(self.chunk, self.N - c * self.chunk))
                for c in range(self.n_chunks)]

    def visible_pairs(self) -> int:
        """Number of visible (query, key) pairs over all heads: key position <= query position
        when causal, every pair otherwise."""
        if not self.causal:
            return self.M * self.N * self.B * self.H
        pos = self.q_pos0 + np.arange(self.M, dtype=np.int64)
        per_head = int(np.minimum(pos + 1, self.N).sum())
        return per_head * self.B * self.H


WORKLOADS = {
    0: Workload(0, "tiny", 1, 4, 256, 256, 0, 64, None),
    1: Workload(1, "incore_m2048", 1, 32, 2048, 2048, 0, 512, None),
    2: Workload(2, "batch8_m2048", 8, 32, 2048, 2048, 0, 512, 16),
    3: Workload(3, "append_133k", 1, 32, 2048, 133120, 131072, 8192, 64),
    4: Workload(4, "stream_1m", 1, 32, 2048, 1048576, 1046528, 16384, 32, streamed=True),
    5: Workload(5, "burst_verify_1m", 1, 32, 64, 1048576, 1048576, 16384, None, streamed=True,
                causal=False),
    6: Workload(6, "layers16_1m", 1, 32, 2048, 1048576, 1046528, 16384, 2, streamed=True,
                layers=16),
}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _fill_slice(out: torch.Tensor, i: int, seed: int) -> None:
    out[i].normal_(generator=_gen(seed * 1_000_003 + i))


def randn(shape, seed: int) -> np.ndarray:
    """float32 N(0, 1) draws of the given shape [..., rows, 64], C-contiguous numpy array."""
    shape = tuple(int(d) for d in shape)
    out = torch.empty(shape, dtype=torch.float32)
    flat = out.view((-1,) + shape[-2:])
    n = flat.shape[0]
    if n == 1 or flat[0].numel() < (1 << 16):
        for i in range(n):
            _fill_slice(flat, i, seed)
    else:
        with ThreadPoolExecutor(max_workers=min(n, _workers())) as ex:
            list(ex.map(lambda i: _fill_slice(flat, i, seed), range(n)))
    return out.numpy()


def _workers() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return 4


def to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Store float32 values as FP16 (round to nearest even); returns the uint16 bit patterns."""
    return np.ascontiguousarray(x.astype(np.float16)).view(np.uint16)


def gen_q(w: Workload, layer: int = 0) -> np.ndarray:
    """Q as FP16 bit patterns, uint16 [B, H, M, 64]."""
    return to_f16_bits(randn((w.B, w.H, w.M, w.D), 1000 * w.wid + 1 + 100_000 * layer))


def gen_kv(w: Workload):
    """Float32 K and V, [B, H, N, 64] each (resident workloads only)."""
    if w.streamed:
        raise ValueError("streamed workloads are drawn per chunk (gen_kv_chunk)")
    shape = (w.B, w.H, w.N, w.D)
    return randn(shape, 1000 * w.wid + 2), randn(shape, 1000 * w.wid + 3)


def gen_kv_chunk(w: Workload, c: int, layer: int = 0):
    """Float32 K and V of chunk c of a streamed workload, [H, n_kv, 64] each (B = 1)."""
    kv_pos0, n_kv = w.chunks()[c]
    shape = (w.H, n_kv, w.D)
    base = 1000 * w.wid + 100_000 * layer
    return (randn(shape, base + 100 + 2 * c),
            randn(shape, base + 101 + 2 * c))


def gen_kv_chunk_head(w: Workload, c: int, h: int, layer: int = 0):
    """Head h of gen_kv_chunk(w, c, layer): the same float32 K and V draws, [n_kv, 64] each, for
    one head only."""
    kv_pos0, n_kv = w.chunks()[c]
    base = 1000 * w.wid + 100_000 * layer
    out = []
    for seed in (base + 100 + 2 * c, base + 101 + 2 * c):
        t = torch.empty((n_kv, w.D), dtype=torch.float32)
        t.normal_(generator=_gen(seed * 1_000_003 + h))
        out.append(t.numpy())
    return out[0], out[1]


def sample_rows(w: Workload, rows_per_head: int | None = None) -> np.ndarray:
    """Flat row ids (b*H + h)*M + i, sorted, for the rows the oracle checks."""
    r = rows_per_head if rows_per_head is not None else w.rows_per_head
    if r is None or r >= w.M:
        return np.arange(w.B * w.H * w.M, dtype=np.int64)
    rng = np.random.default_rng(1000 * w.wid + 9)
    out = []
    for head in range(w.B * w.H):
        pick = rng.choice(np.arange(1, w.M - 1), size=r - 2, replace=False)
        idx = np.concatenate([[0, w.M - 1], pick])
        out.append(head * w.M + np.sort(idx))
    return np.concatenate(out).astype(np.int64)


def small_case(B: int, H: int, M: int, N: int, q_pos0: int, seed: int):
    """A free-form seeded case for parity tests: (Q FP16 bits [B,H,M,64], K, V float32
    [B,H,N,64])."""
    q = to_f16_bits(randn((B, H, M, HEAD_DIM), seed * 10 + 1))
    k = randn((B, H, N, HEAD_DIM), seed * 10 + 2)
    v = randn((B, H, N, HEAD_DIM), seed * 10 + 3)
    return q, k, v
