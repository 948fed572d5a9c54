"""FP64 CPU oracle for chunked causal attention over a Q8_0 KV cache -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package.  It shares no code with the HIP library (``chunked_flashattention_q8_amd``)
and neither imports the other.  The arithmetic lives in ``q8_oracle.c`` (plain C, binary64,
built with gcc); this module only marshals numpy arrays.

What it computes, and where the pages define it:

* ``f32_to_f16`` / ``f16_to_f64`` -- the IEEE binary16 format (the FP16 scale of a Q8_0 block).
* ``q8_0_pack`` / ``q8_0_dequant`` -- block_q8_0 of "Core Architecture & The 4-Brick Pipeline",
  Sec. 5 (Brick 4): 32 int8 values plus an FP16 scale, 34 bytes; two blocks per 64-dim row
  ("Out-of-Core Flash Streaming ...", Sec. 1).
* ``attention`` -- softmax(Q K^T / sqrt(D)) V with the triangular causal mask (Mode A of
  "Out-of-Core Flash Streaming ...", Sec. 4), single pass, plus LSE = m + ln l.
* ``attention_chunks`` -- the chunk recurrence of "Out-of-Core Flash Streaming ...", Sec. 3
  ("Chunked FlashAttention: Exact Mathematical Derivation"), steps 1-6, in the pages' order.
* ``finalize`` -- O / l after the last chunk (same section), and LSE = m + ln l.
* ``kv_bytes`` -- the KV-cache size formulas of the same page, Sec. 1.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "q8_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libq8oracle.so")
# the sanitizer tier (tests/test_sanitizers.py) points this at an instrumented build of the
# same source
_LIB_OVERRIDE = os.environ.get("Q8_ORACLE_LIB")
_lib = None

KV_Q8_0 = 0
KV_F16 = 1
QK = 32
BLOCK_BYTES = 34


def build(force: bool = True) -> str:
    """Compile q8_oracle.c with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
               "-shared", "-pthread", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Problem(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("kv_fmt", ctypes.c_int32), ("B", ctypes.c_int32), ("H", ctypes.c_int32),
                ("M", ctypes.c_int32), ("N", ctypes.c_int32), ("D", ctypes.c_int32),
                ("q_pos0", ctypes.c_int64), ("causal", ctypes.c_int32)]


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE:
        lib = ctypes.CDLL(_LIB_OVERRIDE)
    else:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i64, i32 = ctypes.c_int64, ctypes.c_int32
    lib.orc_f16_to_f64.restype = ctypes.c_double
    lib.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.orc_f32_to_f16.restype = ctypes.c_uint16
    lib.orc_f32_to_f16.argtypes = [ctypes.c_float]
    lib.orc_f32_to_f16_array.argtypes = [P, P, i64]
    lib.orc_f16_to_f64_array.argtypes = [P, P, i64]
    lib.orc_q8_0_pack.restype = i64
    lib.orc_q8_0_pack.argtypes = [P, P, i64, ctypes.c_int]
    lib.orc_q8_0_dequant.argtypes = [P, P, i64]
    lib.orc_attention_rows.restype = ctypes.c_int
    lib.orc_attention_rows.argtypes = [ctypes.POINTER(_Problem), P, i64, P, P, ctypes.c_int]
    lib.orc_attention_chunks.restype = ctypes.c_int
    lib.orc_attention_chunks.argtypes = [ctypes.POINTER(_Problem), P, i64, P, P, ctypes.c_int,
                                         P, P, P, ctypes.c_int]
    lib.orc_finalize.argtypes = [P, P, P, i64, ctypes.c_int, P, P]
    lib.orc_merge_states.argtypes = [P, P, P, P, P, P, i64, ctypes.c_int]
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def default_threads() -> int:
    try:
        return max(1, min(len(os.sched_getaffinity(0)), 64))
    except AttributeError:  # pragma: no cover
        return max(1, min(os.cpu_count() or 1, 64))


# --------------------------------------------------------------------------- binary16 codec

def f32_to_f16(x) -> np.ndarray:
    """float32 array -> binary16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    out = np.empty(x.shape, dtype=np.uint16)
    _load().orc_f32_to_f16_array(_ptr(x), _ptr(out), x.size)
    return out


def f16_to_f64(h) -> np.ndarray:
    """binary16 bit patterns (uint16) -> exact float64 values."""
    h = np.ascontiguousarray(np.asarray(h, dtype=np.uint16))
    out = np.empty(h.shape, dtype=np.float64)
    _load().orc_f16_to_f64_array(_ptr(h), _ptr(out), h.size)
    return out


# --------------------------------------------------------------------------- Q8_0 codec

def q8_0_pack(x, nthreads: int | None = None) -> np.ndarray:
    """float32 [..., L] (L % 32 == 0) -> uint8 [..., L/32*34]: per 32-value block the binary16
    scale (little-endian) then 32 int8 values."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    if x.shape[-1] % QK:
        raise ValueError("last dimension must be a multiple of 32")
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input is outside the Q8_0 codec's domain")
    n_blocks = x.size // QK
    out = np.empty(x.shape[:-1] + (x.shape[-1] // QK * BLOCK_BYTES,), dtype=np.uint8)
    bad = _load().orc_q8_0_pack(_ptr(x), _ptr(out), n_blocks, nthreads or default_threads())
    if bad:
        raise ValueError("%d block(s) have a scale beyond the binary16 range" % bad)
    return out


def q8_0_dequant(b) -> np.ndarray:
    """uint8 [..., L/32*34] -> float64 [..., L], value = q * d16 (exact)."""
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint8))
    if b.shape[-1] % BLOCK_BYTES:
        raise ValueError("last dimension must be a multiple of 34 bytes")
    n_blocks = b.size // BLOCK_BYTES
    out = np.empty(b.shape[:-1] + (b.shape[-1] // BLOCK_BYTES * QK,), dtype=np.float64)
    _load().orc_q8_0_dequant(_ptr(b), _ptr(out), n_blocks)
    return out


# --------------------------------------------------------------------------- attention

@dataclass
class Problem:
    """Q: uint16 binary16 bits [B,H,M,D]; K, V: Q8_0 bytes [B,H,N,D/32*34] (kv_fmt=KV_Q8_0) or
    binary16 bits [B,H,N,D] (kv_fmt=KV_F16).  Query row i sits at position q_pos0 + i, key j at
    position j."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    kv_fmt: int = KV_Q8_0
    q_pos0: int = 0
    causal: bool = True

    def dims(self):
        B, H, M, D = self.q.shape
        N = self.k.shape[2]
        return B, H, M, N, D

    def _struct(self) -> _Problem:
        B, H, M, N, D = self.dims()
        if self.q.dtype != np.uint16 or not self.q.flags["C_CONTIGUOUS"]:
            raise TypeError("q must be C-contiguous uint16 binary16 bits")
        if self.kv_fmt == KV_Q8_0:
            want = (B, H, N, D // QK * BLOCK_BYTES)
            dt = np.uint8
        else:
            want = (B, H, N, D)
            dt = np.uint16
        for name, a in (("k", self.k), ("v", self.v)):
            if a.shape != want or a.dtype != dt or not a.flags["C_CONTIGUOUS"]:
                raise TypeError("%s must be C-contiguous %s of shape %s" % (name, dt, want))
        if D % QK:
            raise ValueError("head dim must be a multiple of 32")
        return _Problem(_ptr(self.q), _ptr(self.k), _ptr(self.v), self.kv_fmt, B, H, M, N, D,
                        int(self.q_pos0), 1 if self.causal else 0)


def _rows_arg(prob: Problem, rows):
    B, H, M, N, D = prob.dims()
    if rows is None:
        rows = np.arange(B * H * M, dtype=np.int64)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    if rows.ndim != 1 or (rows.size and (rows.min() < 0 or rows.max() >= B * H * M)):
        raise ValueError("rows must be flat ids (b*H + h)*M + i")
    if rows.size > 1 and np.any(np.diff(rows // M) < 0):
        raise ValueError("rows must be sorted by head")
    return rows


def attention(prob: Problem, rows=None, nthreads: int | None = None):
    """Single-pass FP64 attention for the given flat rows (default: all).
    Returns (O [n,D] float64, LSE [n] float64)."""
    rows = _rows_arg(prob, rows)
    D = prob.dims()[4]
    st = prob._struct()
    O = np.zeros((rows.size, D), dtype=np.float64)
    lse = np.zeros(rows.size, dtype=np.float64)
    if rows.size:
        rc = _load().orc_attention_rows(ctypes.byref(st), _ptr(rows), rows.size, _ptr(O),
                                        _ptr(lse), nthreads or default_threads())
        if rc:
            raise MemoryError("oracle allocation failed")
    return O, lse


def init_state(n_rows: int, D: int):
    """The empty state: m = -inf, l = 0, O = 0."""
    return (np.full(n_rows, -np.inf), np.zeros(n_rows), np.zeros((n_rows, D)))


def attention_chunks(prob: Problem, chunks, rows=None, state=None,
                     nthreads: int | None = None):
    """Apply the chunk recurrence for each (kv_start, n_kv) in ``chunks`` (in order) to the state
    (m, l, O) of the given rows.  Returns the new (m, l, O) (copies)."""
    rows = _rows_arg(prob, rows)
    B, H, M, N, D = prob.dims()
    c = np.ascontiguousarray(np.asarray(chunks, dtype=np.int64).reshape(-1, 2))
    if c.size and (c[:, 0].min() < 0 or (c[:, 0] + c[:, 1]).max() > N or c[:, 1].min() < 0):
        raise ValueError("chunk outside [0, N)")
    cs = np.ascontiguousarray(c[:, 0])
    cl = np.ascontiguousarray(c[:, 1])
    if state is None:
        state = init_state(rows.size, D)
    m = np.array(state[0], dtype=np.float64, copy=True)
    l = np.array(state[1], dtype=np.float64, copy=True)
    O = np.ascontiguousarray(np.array(state[2], dtype=np.float64, copy=True))
    st = prob._struct()
    if rows.size and len(cs):
        rc = _load().orc_attention_chunks(ctypes.byref(st), _ptr(rows), rows.size, _ptr(cs),
                                          _ptr(cl), len(cs), _ptr(m), _ptr(l), _ptr(O),
                                          nthreads or default_threads())
        if rc:
            raise MemoryError("oracle allocation failed")
    return m, l, O


def merge_states(a, b):
    """Merge partial state b (m, l, O) into a copy of partial state a, both over the same rows
    and disjoint key sets: the state a single pass over both key sets reaches."""
    m = np.array(a[0], dtype=np.float64, copy=True)
    l = np.array(a[1], dtype=np.float64, copy=True)
    O = np.ascontiguousarray(np.array(a[2], dtype=np.float64, copy=True))
    mb = np.ascontiguousarray(np.asarray(b[0], dtype=np.float64))
    lb = np.ascontiguousarray(np.asarray(b[1], dtype=np.float64))
    Ob = np.ascontiguousarray(np.asarray(b[2], dtype=np.float64))
    if mb.shape != m.shape or Ob.shape != O.shape:
        raise ValueError("states of different shapes")
    n, D = O.shape
    _load().orc_merge_states(_ptr(m), _ptr(l), _ptr(O), _ptr(mb), _ptr(lb), _ptr(Ob), n, D)
    return m, l, O


def finalize(m, l, O):
    """O / l and LSE = m + ln l; rows with l = 0 give 0 and -inf."""
    m = np.ascontiguousarray(np.asarray(m, dtype=np.float64))
    l = np.ascontiguousarray(np.asarray(l, dtype=np.float64))
    O = np.ascontiguousarray(np.asarray(O, dtype=np.float64))
    n, D = O.shape
    out = np.empty_like(O)
    lse = np.empty(n, dtype=np.float64)
    _load().orc_finalize(_ptr(m), _ptr(l), _ptr(O), n, D, _ptr(out), _ptr(lse))
    return out, lse


# --------------------------------------------------------------------------- closed forms

def kv_bytes(layers: int, heads: int, tokens: int, head_dim: int, fmt: str) -> int:
    """KV-cache bytes as the formulas of "Out-of-Core Flash Streaming ...", Sec. 1 state them:
    K and V (factor 2) x layers x heads x tokens x bytes per head row, where a row is
    head_dim x 2 bytes in FP16 and head_dim/32 blocks x 34 bytes in Q8_0."""
    if fmt == "f16":
        row = head_dim * 2
    elif fmt == "q8_0":
        if head_dim % QK:
            raise ValueError("head_dim must be a multiple of 32")
        row = head_dim // QK * BLOCK_BYTES
    else:
        raise ValueError(fmt)
    return 2 * layers * heads * tokens * row
