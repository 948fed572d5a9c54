"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every function the
header declares, and each invalid argument is rejected with its status before anything is
enqueued."""
import ctypes
import os
import re

import pytest
import torch

import chunked_flashattention_q8_amd as q8a

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q8attn.h")
NO_GPU = torch.cuda.device_count() == 0

# fake device addresses: never dereferenced, because every call below fails validation first
A16 = 0x10000
A16B = 0x20000
A16C = 0x30000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_and_binding_agree():
    names = declared_functions()
    assert set(names) == set(q8a.EXPORTS), names


def test_library_exports_every_declared_symbol():
    lib = q8a.library()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    assert q8a.status_string(0) == "ok"
    for s in range(1, 7):
        assert q8a.status_string(s) != "unknown status"
    assert q8a.status_string(99) == "unknown status"


def rc_of(fn):
    try:
        fn()
    except q8a.Q8AError as e:
        return e.status
    return q8a.Q8A_OK


def test_pack_rejects_bad_arguments():
    lib = q8a.library()
    P = ctypes.c_void_p
    assert lib.q8_0_pack(P(A16), P(A16B), -1, 64, None) == q8a.Q8A_E_INVAL
    assert lib.q8_0_pack(P(A16), P(A16B), 4, 48, None) == q8a.Q8A_E_INVAL
    assert lib.q8_0_pack(P(A16), P(A16B), 4, 0, None) == q8a.Q8A_E_INVAL
    assert lib.q8_0_pack(None, P(A16B), 4, 64, None) == q8a.Q8A_E_INVAL
    assert lib.q8_0_pack(P(A16 + 4), P(A16B), 4, 64, None) == q8a.Q8A_E_ALIGN
    assert lib.q8_0_pack(P(A16), P(A16B + 1), 4, 64, None) == q8a.Q8A_E_ALIGN
    assert lib.q8_0_pack(P(A16), P(A16B), 0, 64, None) == q8a.Q8A_OK  # nothing to do
    assert lib.q8_0_pack(P(A16), P(A16B), (1 << 27) + 1, 64, None) == q8a.Q8A_E_INVAL


def test_state_init_rejects_bad_arguments():
    lib = q8a.library()
    st = q8a.q8a_state()
    P = ctypes.c_void_p
    ok = (P(A16), P(A16B), P(A16C))
    assert lib.attn_state_init(ctypes.byref(st), *ok, 1, 4, 256, 128, 0, None) == \
        q8a.Q8A_E_UNSUPPORTED
    assert lib.attn_state_init(ctypes.byref(st), *ok, 0, 4, 256, 64, 0, None) == q8a.Q8A_E_INVAL
    assert lib.attn_state_init(ctypes.byref(st), *ok, 1, 4, 256, 64, -1, None) == \
        q8a.Q8A_E_INVAL
    assert lib.attn_state_init(ctypes.byref(st), P(A16), P(A16B), P(A16C + 8), 1, 4, 256, 64,
                               0, None) == q8a.Q8A_E_ALIGN
    assert lib.attn_state_init(None, *ok, 1, 4, 256, 64, 0, None) == q8a.Q8A_E_INVAL
    assert lib.attn_state_init(ctypes.byref(st), *ok, 1, 1, 1 << 24, 64, 0, None) == \
        q8a.Q8A_E_UNSUPPORTED                                  # beyond 32-bit row offsets
    assert lib.attn_state_init(ctypes.byref(st), *ok, 4096, 4096, 1, 64, 0, None) == \
        q8a.Q8A_E_UNSUPPORTED                                  # 2^24 (sequence, head) pairs
    assert lib.attn_state_init(ctypes.byref(st), *ok, 64, 64, 1 << 17, 64, 0, None) == \
        q8a.Q8A_E_UNSUPPORTED                                  # 2^29 rows
    assert st.magic == 0  # untouched on failure


def fake_state(B=1, H=4, M=256):
    st = q8a.q8a_state()
    st.m, st.l, st.o = A16, A16B, A16C
    st.n_seq, st.n_heads, st.n_q, st.head_dim = B, H, M, 64
    st.q_pos0 = 0
    st.magic = q8a.STATE_MAGIC
    return st


def acc(st, q=A16, k=A16B, v=A16C, dtype=0, pos=0, n=64, hs=None, ss=0, causal=1):
    if hs is None:
        hs = 256 * 68
    P = ctypes.c_void_p
    return q8a.library().attn_accumulate_chunk(ctypes.byref(st), P(q), P(k), P(v), dtype, pos,
                                               n, hs, ss, causal, None)


def test_accumulate_rejects_bad_arguments():
    st = fake_state()
    assert acc(q8a.q8a_state()) == q8a.Q8A_E_STATE          # not initialised
    bad = fake_state()
    bad.head_dim = 128
    assert acc(bad) == q8a.Q8A_E_STATE
    assert acc(st, dtype=7) == q8a.Q8A_E_INVAL
    assert acc(st, n=0) == q8a.Q8A_E_INVAL
    assert acc(st, pos=-1) == q8a.Q8A_E_INVAL
    assert acc(st, causal=2) == q8a.Q8A_E_INVAL
    assert acc(st, q=0) == q8a.Q8A_E_INVAL
    assert acc(st, hs=64 * 68 - 16) == q8a.Q8A_E_INVAL      # head stride shorter than a chunk
    assert acc(st, hs=-16) == q8a.Q8A_E_INVAL
    assert acc(st, n=40_000_000) == q8a.Q8A_E_INVAL         # beyond the 32-bit byte range
    assert acc(st, k=A16B + 4) == q8a.Q8A_E_ALIGN
    assert acc(st, q=A16 + 8) == q8a.Q8A_E_ALIGN
    assert acc(st, hs=256 * 68 + 4) == q8a.Q8A_E_ALIGN
    st2 = fake_state(B=2)
    assert acc(st2, ss=0) == q8a.Q8A_E_INVAL                # sequences would overlap


K_NEW, V_NEW, K_CACHE, V_CACHE = 0x1000000, 0x2000000, 0x3000000, 0x4000000


def append(st, q=A16, kn=K_NEW, vn=V_NEW, kc=K_CACHE, vc=V_CACHE, pos=0, n=64, hs=None, ss=0,
           causal=1):
    if hs is None:
        hs = 256 * 68
    P = ctypes.c_void_p
    return q8a.library().attn_append_chunk(ctypes.byref(st), P(q), P(kn), P(vn), P(kc), P(vc),
                                           pos, n, hs, ss, causal, None)


def test_append_rejects_bad_arguments():
    st = fake_state()
    assert append(q8a.q8a_state()) == q8a.Q8A_E_STATE        # not initialised
    assert append(st, kn=0) == q8a.Q8A_E_INVAL
    assert append(st, vn=0) == q8a.Q8A_E_INVAL
    assert append(st, kc=0) == q8a.Q8A_E_INVAL
    assert append(st, n=0) == q8a.Q8A_E_INVAL
    assert append(st, causal=3) == q8a.Q8A_E_INVAL
    assert append(st, kn=K_NEW + 4) == q8a.Q8A_E_ALIGN
    assert append(st, vc=V_CACHE + 4) == q8a.Q8A_E_ALIGN
    assert append(st, hs=64 * 68 - 16) == q8a.Q8A_E_INVAL     # heads' runs would overlap
    assert append(st, hs=1 << 47) == q8a.Q8A_E_INVAL          # stride out of range
    assert append(st, vc=K_CACHE + 4096) == q8a.Q8A_E_INVAL   # K and V destinations overlap
    assert append(st, kc=K_NEW + 1024) == q8a.Q8A_E_INVAL     # destination over a source
    assert append(st, vc=V_NEW) == q8a.Q8A_E_INVAL
    st2 = fake_state(B=2)
    # sequence stride inside the head runs: (seq 1, head 0) would land on (seq 0, head 1)
    assert append(st2, hs=64 * 68, ss=64 * 68) == q8a.Q8A_E_INVAL
    assert append(st2, hs=64 * 68, ss=0) == q8a.Q8A_E_INVAL
    big = fake_state(B=300, H=300)
    assert append(big, hs=64 * 68, ss=300 * 64 * 68) == q8a.Q8A_E_UNSUPPORTED
    assert append(st, kc=A16) == q8a.Q8A_E_INVAL                # over Q (and the state's m)
    assert append(st, vc=A16C) == q8a.Q8A_E_INVAL               # over the state's O
    tall = fake_state(H=1, M=1 << 24)
    assert acc(tall) == q8a.Q8A_E_UNSUPPORTED


@pytest.mark.skipif(not NO_GPU, reason="needs a host without a GPU")
def test_append_valid_layouts_pass_validation():
    """Heads outside sequences and sequences outside heads are both accepted (validation passes
    and the launch then fails for want of a device)."""
    st2 = fake_state(B=2)
    assert append(st2, hs=64 * 68, ss=4 * 64 * 68) == q8a.Q8A_E_HIP
    assert append(st2, hs=2 * 64 * 68, ss=64 * 68) == q8a.Q8A_E_HIP


def acc_final(st, q=0x3000000, k=0x4000000, v=0x5000000, out=0x1000000, lse=0x2000000,
              pos=0, n=64, causal=1):
    P = ctypes.c_void_p
    return q8a.library().attn_accumulate_chunk_final(
        ctypes.byref(st), P(q), P(k), P(v), 0, pos, n, 256 * 68, 0, causal, P(out),
        P(lse) if lse else None, None)


def separate_state():
    st = fake_state()
    st.m, st.l, st.o = 0x6000000, 0x7000000, 0x8000000
    return st


def test_accumulate_final_rejects_bad_arguments():
    st = separate_state()
    assert acc_final(q8a.q8a_state()) == q8a.Q8A_E_STATE       # not initialised
    assert acc_final(st, n=0) == q8a.Q8A_E_INVAL                # the chunk checks apply
    assert acc_final(st, causal=0) == q8a.Q8A_E_INVAL           # final rows need the causal mask
    assert acc_final(st, out=0) == q8a.Q8A_E_INVAL
    assert acc_final(st, out=0x1000000 + 8) == q8a.Q8A_E_ALIGN
    assert acc_final(st, lse=0x2000000 + 2) == q8a.Q8A_E_ALIGN
    assert acc_final(st, out=0x3000000 + 4096) == q8a.Q8A_E_INVAL   # out over Q
    assert acc_final(st, out=0x8000000) == q8a.Q8A_E_INVAL          # out over the state's O
    assert acc_final(st, lse=0x6000000) == q8a.Q8A_E_INVAL          # lse over the state's m
    assert acc_final(st, lse=0x1000000 + 1024) == q8a.Q8A_E_INVAL   # lse over out
    assert acc_final(st, out=0x4000000 - 64) == q8a.Q8A_E_INVAL     # out runs into K


@pytest.mark.skipif(not NO_GPU, reason="needs a host without a GPU")
def test_accumulate_final_valid_arguments_pass_validation():
    st = separate_state()
    assert acc_final(st) == q8a.Q8A_E_HIP
    assert acc_final(st, lse=0) == q8a.Q8A_E_HIP


def test_finalize_rejects_bad_arguments():
    lib = q8a.library()
    P = ctypes.c_void_p
    st = fake_state()
    assert lib.attn_finalize(ctypes.byref(q8a.q8a_state()), P(A16), None, None) == \
        q8a.Q8A_E_STATE
    assert lib.attn_finalize(ctypes.byref(st), None, None, None) == q8a.Q8A_E_INVAL
    assert lib.attn_finalize(ctypes.byref(st), P(A16 + 2), None, None) == q8a.Q8A_E_ALIGN
    assert lib.attn_finalize(ctypes.byref(st), P(A16), P(A16B + 1), None) == q8a.Q8A_E_ALIGN


def test_merge_rejects_bad_arguments():
    lib = q8a.library()

    def merge(a, b):
        return lib.attn_state_merge(ctypes.byref(a), ctypes.byref(b), None)
    a = fake_state()
    b = fake_state()
    b.m, b.l, b.o = 0x110000, 0x120000, 0x200000
    assert merge(q8a.q8a_state(), b) == q8a.Q8A_E_STATE       # dst not initialised
    assert merge(a, q8a.q8a_state()) == q8a.Q8A_E_STATE       # src not initialised
    for field, value in (("n_q", 128), ("n_heads", 2), ("n_seq", 2), ("q_pos0", 5)):
        c = fake_state()
        c.m, c.l, c.o = b.m, b.l, b.o
        setattr(c, field, value)
        assert merge(a, c) == q8a.Q8A_E_STATE, field
    assert merge(a, a) == q8a.Q8A_E_INVAL                     # a state with itself
    c = fake_state()
    c.m, c.l, c.o = b.m, b.l, A16C + 64                       # O buffers overlap
    assert merge(a, c) == q8a.Q8A_E_INVAL


def test_stream_rejects_bad_arguments():
    lib = q8a.library()
    P = ctypes.c_void_p
    st = fake_state(H=2, M=64)
    slots = (P * 2)(A16B, A16C)
    slots_bad = (P * 2)(A16B, None)
    args = dict(q=P(A16), kh=P(0x40000), vh=P(0x50000))

    def call(st_, sk, sv, n_total=1000, chunk=256, dtype=0):
        return lib.attn_accumulate_stream(ctypes.byref(st_), args["q"], args["kh"], args["vh"],
                                          dtype, n_total, chunk, sk, sv, 1, None, None)
    assert call(st, slots, slots_bad) == q8a.Q8A_E_INVAL
    assert call(st, slots, slots, n_total=0) == q8a.Q8A_E_INVAL
    assert call(st, slots, slots, chunk=0) == q8a.Q8A_E_INVAL
    assert call(q8a.q8a_state(), slots, slots) == q8a.Q8A_E_STATE
    assert call(st, slots, slots, dtype=3) == q8a.Q8A_E_INVAL
    assert call(st, (P * 2)(A16B, A16C + 8), slots) == q8a.Q8A_E_ALIGN


def test_file_feed_rejects_bad_arguments():
    lib = q8a.library()
    P = ctypes.c_void_p
    st = fake_state(H=2, M=64)
    chunk = 256
    cb = 2 * chunk * 68                       # chunk bytes (one sequence, two heads)
    slots = (P * 2)(A16B, A16C)
    ring = (P * 2)(0x1000000, 0x2000000)      # 4096-aligned fake host addresses
    ring2 = (P * 2)(0x3000000, 0x4000000)

    def call(st_=st, fk=3, fv=4, off=0, rk=ring, rv=ring2, rb=cb + 8192, sk=slots, sv=slots,
             n_total=1000, dtype=0):
        return lib.attn_accumulate_file(ctypes.byref(st_), P(A16), fk, fv, off, dtype, n_total,
                                        chunk, rk, rv, rb, sk, sv, 1, None, None)
    assert call(fk=-1) == q8a.Q8A_E_INVAL
    assert call(fv=-5) == q8a.Q8A_E_INVAL
    assert call(off=-1) == q8a.Q8A_E_INVAL
    assert call(n_total=0) == q8a.Q8A_E_INVAL
    assert call(rk=(P * 2)(0x1000000, None)) == q8a.Q8A_E_INVAL
    assert call(rb=cb + 8191) == q8a.Q8A_E_INVAL             # no room for the aligned read
    assert call(rv=(P * 2)(0x3000000, 0x4000000 + 2048)) == q8a.Q8A_E_ALIGN
    assert call(sk=(P * 2)(A16B, A16C + 8)) == q8a.Q8A_E_ALIGN
    assert call(st_=q8a.q8a_state()) == q8a.Q8A_E_STATE
    assert call(dtype=4) == q8a.Q8A_E_INVAL


@pytest.mark.skipif(not NO_GPU, reason="needs a host without a GPU")
def test_valid_call_without_device_reports_hip_error():
    """On a host with no GPU, a call that passes validation fails in the HIP runtime and says so
    (Q8A_E_HIP plus the hipError_t), instead of falling back to the CPU."""
    lib = q8a.library()
    P = ctypes.c_void_p
    rc = lib.q8_0_pack(P(A16), P(A16B), 4, 64, None)
    assert rc == q8a.Q8A_E_HIP
    assert lib.q8a_last_hip_error() != 0


def test_binding_refuses_views_with_gaps():
    """q8_0_pack writes n_rows dense rows: a strided view (a partial chunk of a cache laid out
    with a larger head stride) is refused by the binding instead of being written past."""
    cache = torch.zeros((2, 10, 68), dtype=torch.uint8)
    x = torch.zeros((2, 6, 64), dtype=torch.float32)
    with pytest.raises(ValueError):
        q8a.q8_0_pack(x, cache[:, :6], 12, 64)
    with pytest.raises(ValueError):
        q8a.q8_0_pack(x.transpose(0, 1), cache, 12, 64)


def test_deferred_init_enqueues_nothing_and_checks_like_init():
    """attn_state_init_deferred takes attn_state_init's checks and fills the descriptor with
    Q8A_STATE_FRESH without touching the device: it succeeds on a host without a GPU."""
    lib = q8a.library()
    P = ctypes.c_void_p
    st = q8a.q8a_state()
    ok = (P(A16), P(A16B), P(A16C))
    assert lib.attn_state_init_deferred(ctypes.byref(st), *ok, 1, 4, 256, 128, 0) == \
        q8a.Q8A_E_UNSUPPORTED
    assert lib.attn_state_init_deferred(ctypes.byref(st), *ok, 0, 4, 256, 64, 0) == \
        q8a.Q8A_E_INVAL
    assert lib.attn_state_init_deferred(ctypes.byref(st), P(A16), P(A16B), P(A16C + 8), 1, 4,
                                        256, 64, 0) == q8a.Q8A_E_ALIGN
    assert lib.attn_state_init_deferred(ctypes.byref(st), *ok, 1, 1, 1 << 24, 64, 0) == \
        q8a.Q8A_E_UNSUPPORTED
    assert st.magic == 0
    assert lib.attn_state_init_deferred(ctypes.byref(st), *ok, 2, 4, 256, 64, 7) == q8a.Q8A_OK
    assert st.magic == q8a.STATE_MAGIC and st.flags == q8a.STATE_FRESH
    assert (st.m, st.l, st.o, st.n_seq, st.n_heads, st.n_q, st.q_pos0) == \
        (A16, A16B, A16C, 2, 4, 256, 7)


def test_hand_edited_descriptor_sizes_are_rejected():
    """A descriptor with sizes attn_state_init refuses as unsupported (edited by hand after
    init) is refused the same way by every call that reads it, before anything is enqueued."""
    for B, H, M in ((65535, 200, 1), (4096, 4096, 1), (1, 64, (1 << 23) + 1), (1, 1, 1 << 24)):
        st = fake_state(B=B, H=H, M=M)
        assert acc(st, ss=256 * 68 * H) == q8a.Q8A_E_UNSUPPORTED, (B, H, M)
        assert q8a.library().attn_finalize(ctypes.byref(st), ctypes.c_void_p(A16), None,
                                           None) == q8a.Q8A_E_UNSUPPORTED, (B, H, M)


def test_unknown_state_flags_are_rejected():
    st = fake_state()
    st.flags = 0x100
    assert acc(st) == q8a.Q8A_E_STATE
    for form in (0x50, 0x60, 0x70):  # reserved tile forms
        st.flags = form
        assert acc(st) == q8a.Q8A_E_STATE
    assert q8a.library().attn_finalize(ctypes.byref(st), ctypes.c_void_p(A16), None, None) == \
        q8a.Q8A_E_STATE


@pytest.mark.skipif(not NO_GPU, reason="needs a host without a GPU")
def test_fresh_bit_survives_a_failed_launch():
    """A call on a FRESH state clears the bit only once its work is enqueued: with no device
    the launch fails (Q8A_E_HIP) and the bit stays set, for every entry point that reads the
    state; a FRESH src merges as a no-op."""
    lib = q8a.library()
    P = ctypes.c_void_p
    for first_pos in (0, 300):  # every row sees the chunk / the initialisation comes first
        st = separate_state()
        st.flags = q8a.STATE_FRESH | q8a.FORM_NARROW
        assert acc(st, pos=first_pos) == q8a.Q8A_E_HIP
        assert st.flags == q8a.STATE_FRESH | q8a.FORM_NARROW
        assert acc_final(st, pos=first_pos) == q8a.Q8A_E_HIP
        assert st.flags & q8a.STATE_FRESH
    st = fake_state()
    st.flags = q8a.STATE_FRESH
    assert lib.attn_finalize(ctypes.byref(st), P(0x9000000), None, None) == q8a.Q8A_E_HIP
    assert st.flags == q8a.STATE_FRESH
    a = fake_state()
    b = fake_state()
    b.m, b.l, b.o = 0x110000, 0x120000, 0x200000
    b.flags = q8a.STATE_FRESH
    assert lib.attn_state_merge(ctypes.byref(a), ctypes.byref(b), None) == q8a.Q8A_OK
    a.flags = q8a.STATE_FRESH
    b.flags = 0
    assert lib.attn_state_merge(ctypes.byref(a), ctypes.byref(b), None) == q8a.Q8A_E_HIP
    assert a.flags == q8a.STATE_FRESH


def test_sub_state_of_a_deferred_state_is_refused():
    st = fake_state(B=2)
    st.flags = q8a.STATE_FRESH
    with pytest.raises(ValueError):
        q8a.sub_state(st, 1, 1)
