"""Python binding of libq8attn.so: exact chunked causal attention prefill over a Q8_0 KV cache
on AMD MI355X (gfx950).

Argument marshalling only.  Every step of the computation runs in the HIP kernels behind the C
ABI declared in ``include/q8attn.h``; PyTorch supplies device memory and streams.  The names and
arguments mirror the C functions; tensors are accepted wherever the C function takes a pointer
(raw integer addresses are accepted too).  If the shared library is not built, importing works
but every call raises: there is no CPU fallback.

The method ("Out-of-Core Flash Streaming & Speculative Decode (1M Context)", Sec. 3): the KV
sequence is consumed in chunks while the online-softmax state (m, l, unnormalised O) of every
query row persists across the calls, so O / l after the last chunk equals single-pass softmax
attention.  Q8_0 is block_q8_0 of "Core Architecture & The 4-Brick Pipeline", Sec. 5.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libq8attn.so")

Q8A_OK = 0
Q8A_E_INVAL = 1
Q8A_E_UNSUPPORTED = 2
Q8A_E_ALIGN = 3
Q8A_E_STATE = 4
Q8A_E_HIP = 5
Q8A_E_IO = 6
KV_Q8_0 = 0
KV_F16 = 1
STATE_MAGIC = 0x51384154
# bits of q8a_state.flags (include/q8attn.h)
STATE_FRESH = 0x1
STATE_FINAL_OUT_ONLY = 0x2
FORM_MASK = 0x70
FORM_AUTO = 0x00
FORM_WIDE = 0x10
FORM_NARROW = 0x20
FORM_KEY_SPLIT = 0x30
FORM_SPLIT = 0x40
HEAD_DIM = 64
ROW_BYTES = {KV_Q8_0: 68, KV_F16: 128}

EXPORTS = ("q8_0_pack", "attn_state_init", "attn_state_init_deferred", "attn_accumulate_chunk",
           "attn_accumulate_chunk_final", "attn_append_chunk",
           "attn_finalize",
           "attn_state_merge", "attn_accumulate_stream", "attn_accumulate_file",
           "q8a_status_string",
           "q8a_last_hip_error")


class Q8AError(RuntimeError):
    def __init__(self, status: int, hip_error: int = 0):
        self.status = status
        self.hip_error = hip_error
        msg = "%s (status %d)" % (status_string(status), status)
        if status == Q8A_E_HIP:
            msg += ", hipError_t %d" % hip_error
        super().__init__(msg)


class q8a_state(ctypes.Structure):
    """Mirror of the C descriptor q8a_state."""
    _fields_ = [("m", ctypes.c_void_p), ("l", ctypes.c_void_p), ("o", ctypes.c_void_p),
                ("n_seq", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("n_q", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("q_pos0", ctypes.c_int64), ("magic", ctypes.c_uint32),
                ("flags", ctypes.c_uint32)]


_lib = None


def library() -> ctypes.CDLL:
    """The loaded libq8attn.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libq8attn.so is not built (run __graft_entry__.build()); "
                           "there is no CPU fallback")
    lib = ctypes.CDLL(LIB_PATH)
    P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    SP = ctypes.POINTER(q8a_state)
    lib.q8_0_pack.argtypes = [P, P, i64, i32, P]
    lib.attn_state_init.argtypes = [SP, P, P, P, i32, i32, i32, i32, i64, P]
    lib.attn_state_init_deferred.argtypes = [SP, P, P, P, i32, i32, i32, i32, i64]
    lib.attn_accumulate_chunk.argtypes = [SP, P, P, P, i32, i64, i32, i64, i64, i32, P]
    lib.attn_accumulate_chunk_final.argtypes = [SP, P, P, P, i32, i64, i32, i64, i64, i32, P,
                                                P, P]
    lib.attn_append_chunk.argtypes = [SP, P, P, P, P, P, i64, i32, i64, i64, i32, P]
    lib.attn_finalize.argtypes = [SP, P, P, P]
    lib.attn_state_merge.argtypes = [SP, SP, P]
    lib.attn_accumulate_stream.argtypes = [SP, P, P, P, i32, i64, i32, ctypes.POINTER(P),
                                           ctypes.POINTER(P), i32, P, P]
    lib.attn_accumulate_file.argtypes = [SP, P, ctypes.c_int, ctypes.c_int, i64, i32, i64, i32,
                                         ctypes.POINTER(P), ctypes.POINTER(P), i64,
                                         ctypes.POINTER(P), ctypes.POINTER(P), i32, P, P]
    lib.q8a_status_string.restype = ctypes.c_char_p
    lib.q8a_status_string.argtypes = [ctypes.c_int]
    lib.q8a_last_hip_error.restype = ctypes.c_int
    lib.q8a_last_hip_error.argtypes = []
    for name in ("q8_0_pack", "attn_state_init", "attn_state_init_deferred",
                 "attn_accumulate_chunk", "attn_append_chunk",
                 "attn_finalize", "attn_state_merge", "attn_accumulate_stream",
                 "attn_accumulate_file"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return library().q8a_status_string(int(status)).decode()


def _check(rc: int) -> None:
    if rc != Q8A_OK:
        raise Q8AError(rc, library().q8a_last_hip_error() if rc == Q8A_E_HIP else 0)


def _ptr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return x.data_ptr()
    if hasattr(x, "__array_interface__"):  # a numpy array (e.g. an mmap'd ring buffer)
        return x.__array_interface__["data"][0]
    return int(x)


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def q8_0_pack(x, dst, n_rows: int, row_len: int, stream=None) -> None:
    """FP32 [n_rows][row_len] -> Q8_0 bytes (n_rows * row_len/32 * 34), on the GPU.  Both
    buffers are dense: a tensor view with gaps (e.g. a partial chunk of a strided cache) is
    refused rather than written past its gaps."""
    for t in (x, dst):
        if isinstance(t, torch.Tensor) and not t.is_contiguous():
            raise ValueError("q8_0_pack takes dense buffers; pack into a contiguous tensor "
                             "and copy it into the strided view")
    _check(library().q8_0_pack(_ptr(x), _ptr(dst), int(n_rows), int(row_len), _stream(stream)))


def attn_state_init(m, l, o, n_seq: int, n_heads: int, n_q: int, head_dim: int, q_pos0: int,
                    stream=None) -> q8a_state:
    """Describe the state buffers and mark every row empty (m = -inf, l = 0)."""
    st = q8a_state()
    _check(library().attn_state_init(ctypes.byref(st), _ptr(m), _ptr(l), _ptr(o), int(n_seq),
                                     int(n_heads), int(n_q), int(head_dim), int(q_pos0),
                                     _stream(stream)))
    return st


def attn_state_init_deferred(m, l, o, n_seq: int, n_heads: int, n_q: int, head_dim: int,
                             q_pos0: int, flags: int = 0) -> q8a_state:
    """Describe the state buffers without enqueueing anything (flags = STATE_FRESH): the first
    call that reads the state initialises it.  `flags` adds further q8a_state.flags bits."""
    st = q8a_state()
    _check(library().attn_state_init_deferred(ctypes.byref(st), _ptr(m), _ptr(l), _ptr(o),
                                              int(n_seq), int(n_heads), int(n_q),
                                              int(head_dim), int(q_pos0)))
    st.flags |= int(flags)
    return st


def set_flags(st: q8a_state, flags: int) -> q8a_state:
    """Set q8a_state.flags bits (STATE_FINAL_OUT_ONLY, a FORM_* tile form) on a descriptor;
    FORM_* bits replace the tile form already set."""
    if flags & FORM_MASK:
        st.flags &= ~FORM_MASK
    st.flags |= int(flags)
    return st


def attn_accumulate_chunk(st: q8a_state, q, k, v, kv_dtype: int, kv_pos0: int, n_kv: int,
                          kv_head_stride: int, kv_seq_stride: int, causal: int = 1,
                          stream=None) -> None:
    """Fold one KV chunk (keys at positions kv_pos0 .. kv_pos0 + n_kv - 1) into the state."""
    _check(library().attn_accumulate_chunk(ctypes.byref(st), _ptr(q), _ptr(k), _ptr(v),
                                           int(kv_dtype), int(kv_pos0), int(n_kv),
                                           int(kv_head_stride), int(kv_seq_stride),
                                           int(causal), _stream(stream)))


def attn_accumulate_chunk_final(st: q8a_state, q, k, v, kv_dtype: int, kv_pos0: int, n_kv: int,
                                kv_head_stride: int, kv_seq_stride: int, out, lse=None,
                                causal: int = 1, stream=None) -> None:
    """attn_accumulate_chunk, plus out/lse of the rows whose query position lies in the chunk
    (final in a causal pass over chunks in ascending key order)."""
    _check(library().attn_accumulate_chunk_final(ctypes.byref(st), _ptr(q), _ptr(k), _ptr(v),
                                                 int(kv_dtype), int(kv_pos0), int(n_kv),
                                                 int(kv_head_stride), int(kv_seq_stride),
                                                 int(causal), _ptr(out), _ptr(lse),
                                                 _stream(stream)))


def attn_append_chunk(st: q8a_state, q, k_new, v_new, k_cache, v_cache, kv_pos0: int, n_kv: int,
                      kv_head_stride: int, kv_seq_stride: int, causal: int = 1,
                      stream=None) -> None:
    """Pack n_kv new FP32 K/V tokens into the Q8_0 cache rows at k_cache / v_cache and fold
    them into the state (the same bytes and state as q8_0_pack + attn_accumulate_chunk)."""
    _check(library().attn_append_chunk(ctypes.byref(st), _ptr(q), _ptr(k_new), _ptr(v_new),
                                       _ptr(k_cache), _ptr(v_cache), int(kv_pos0), int(n_kv),
                                       int(kv_head_stride), int(kv_seq_stride), int(causal),
                                       _stream(stream)))


def attn_finalize(st: q8a_state, out, lse=None, stream=None) -> None:
    """out = O / l (FP16), lse = m + ln l (FP32)."""
    _check(library().attn_finalize(ctypes.byref(st), _ptr(out), _ptr(lse), _stream(stream)))


def attn_state_merge(dst: q8a_state, src: q8a_state, stream=None) -> None:
    """Merge partial state src (a disjoint key set, same rows) into dst."""
    _check(library().attn_state_merge(ctypes.byref(dst), ctypes.byref(src), _stream(stream)))


def attn_accumulate_stream(st: q8a_state, q, k_host, v_host, kv_dtype: int, n_kv_total: int,
                           chunk_tokens: int, slot_k, slot_v, causal: int = 1,
                           compute_stream=None, copy_stream=None) -> None:
    """Stream a chunk-major pinned host KV cache through two device slots per tensor."""
    sk = (ctypes.c_void_p * 2)(_ptr(slot_k[0]), _ptr(slot_k[1]))
    sv = (ctypes.c_void_p * 2)(_ptr(slot_v[0]), _ptr(slot_v[1]))
    _check(library().attn_accumulate_stream(ctypes.byref(st), _ptr(q), _ptr(k_host),
                                            _ptr(v_host), int(kv_dtype), int(n_kv_total),
                                            int(chunk_tokens), sk, sv, int(causal),
                                            _stream(compute_stream), _stream(copy_stream)))


def attn_accumulate_file(st: q8a_state, q, fd_k: int, fd_v: int, file_offset: int, kv_dtype: int,
                         n_kv_total: int, chunk_tokens: int, ring_k, ring_v, ring_bytes: int,
                         slot_k, slot_v, causal: int = 1, compute_stream=None,
                         copy_stream=None) -> None:
    """Stream a chunk-major KV cache from two files (pread into a pinned two-slot ring, then
    through two device slots per tensor); blocks the host until every chunk has been read."""
    rk = (ctypes.c_void_p * 2)(_ptr(ring_k[0]), _ptr(ring_k[1]))
    rv = (ctypes.c_void_p * 2)(_ptr(ring_v[0]), _ptr(ring_v[1]))
    sk = (ctypes.c_void_p * 2)(_ptr(slot_k[0]), _ptr(slot_k[1]))
    sv = (ctypes.c_void_p * 2)(_ptr(slot_v[0]), _ptr(slot_v[1]))
    _check(library().attn_accumulate_file(ctypes.byref(st), _ptr(q), int(fd_k), int(fd_v),
                                          int(file_offset), int(kv_dtype), int(n_kv_total),
                                          int(chunk_tokens), rk, rv, int(ring_bytes), sk, sv,
                                          int(causal), _stream(compute_stream),
                                          _stream(copy_stream)))


def alloc_ring(n_bytes: int, pinned: bool = False):
    """Convenience: the two 4096-byte-aligned host buffers of n_bytes of attn_accumulate_file's
    ring; anonymous mmap memory (for O_DIRECT descriptors, which cannot read into pinned memory)
    or pinned memory (for buffered descriptors)."""
    import mmap

    import numpy as np
    out = []
    for _ in range(2):
        if pinned:
            t = torch.empty(n_bytes + 4096, dtype=torch.uint8, pin_memory=True)
            pad = (-t.data_ptr()) % 4096
            out.append(t[pad:pad + n_bytes])
        else:
            out.append(np.frombuffer(mmap.mmap(-1, n_bytes), dtype=np.uint8))
    return out


def sub_state(st: q8a_state, s0: int, n: int) -> q8a_state:
    """Descriptor of sequences [s0, s0 + n) of an initialised state (same buffers)."""
    if not (0 <= s0 and n >= 1 and s0 + n <= st.n_seq):
        raise ValueError("sequence range outside the state")
    if st.flags & STATE_FRESH:
        raise ValueError("take sub-states of an initialised state, not a deferred one")
    sub = q8a_state()
    ctypes.memmove(ctypes.byref(sub), ctypes.byref(st), ctypes.sizeof(q8a_state))
    rows = s0 * st.n_heads * st.n_q
    sub.m = st.m + 4 * rows
    sub.l = st.l + 4 * rows
    sub.o = st.o + 4 * HEAD_DIM * rows
    sub.n_seq = n
    return sub


def alloc_state(n_seq: int, n_heads: int, n_q: int, device="cuda"):
    """Convenience: FP32 tensors m, l [n_seq,n_heads,n_q] and o [...,64] for a state."""
    m = torch.empty((n_seq, n_heads, n_q), dtype=torch.float32, device=device)
    l = torch.empty_like(m)
    o = torch.empty((n_seq, n_heads, n_q, HEAD_DIM), dtype=torch.float32, device=device)
    return m, l, o
