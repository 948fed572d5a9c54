"""Helpers for the GPU parity tests: run the HIP path through the C ABI and compare with the
oracle at the tolerances of the method's contract:

* O: max |O_gpu - O_ref| <= 2e-3 and ||O_gpu - O_ref||_2 / ||O_ref||_2 <= 1e-3 over every
  checked element, with O_ref the unrounded FP64 oracle value and O_gpu the FP16 output;
* LSE = m + ln l: |LSE_gpu - LSE_ref| <= 1e-4 * max(1, |LSE_ref|) (relative, with an absolute
  floor of 1e-4 where LSE_ref is near 0).
"""
import sys

import numpy as np
import torch

import chunked_flashattention_q8_amd as q8a

MAX_ABS = 2e-3
REL_RMS = 1e-3
LSE_REL = 1e-4
D = 64

# the accumulate kernel's tile form, set in the flags of every state new_state describes (the
# rows_per_workgroup fixture runs a test under each forced form)
FORMS = {"auto": q8a.FORM_AUTO, "128": q8a.FORM_NARROW, "256": q8a.FORM_WIDE,
         "256k": q8a.FORM_KEY_SPLIT, "64": q8a.FORM_SPLIT}
TILE_FORM = [q8a.FORM_AUTO]


def new_state(B, H, M, q_pos0, deferred=False, flags=0):
    """Allocate and describe a state (attn_state_init, or attn_state_init_deferred), with the
    current TILE_FORM and any further flags set.  Returns (st, (m, l, o))."""
    m, l, o = q8a.alloc_state(B, H, M)
    if deferred:
        st = q8a.attn_state_init_deferred(m, l, o, B, H, M, D, q_pos0)
    else:
        st = q8a.attn_state_init(m, l, o, B, H, M, D, q_pos0)
    q8a.set_flags(st, TILE_FORM[0] | flags)
    return st, (m, l, o)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def f16_to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.float16).to(dev())


def gpu_pack(x: np.ndarray) -> torch.Tensor:
    """float32 [..., 64] -> Q8_0 bytes [..., 68] on the GPU via q8_0_pack."""
    xt = torch.from_numpy(np.ascontiguousarray(x)).to(dev())
    out = torch.empty(x.shape[:-1] + (68,), dtype=torch.uint8, device=dev())
    q8a.q8_0_pack(xt, out, x.size // 64, 64)
    return out


def prefill(q, k, v, kv_dtype, B, H, M, N, q_pos0, chunks, causal=1, on_state=None,
            state=None, finalize=True):
    """init -> one attn_accumulate_chunk per (kv_pos0, n_kv) -> finalize, on the current stream.
    k, v: device tensors [B, H, N, row] (bytes) or [B, H, N, 64] FP16.  Returns (out, lse,
    (m, l, o)) as device tensors (out and lse None without the finalize)."""
    row = q8a.ROW_BYTES[kv_dtype]
    if state is None:
        st, (m, l, o) = new_state(B, H, M, q_pos0)
    else:
        st, (m, l, o) = state
    kp, vp = k.data_ptr(), v.data_ptr()
    for (s, n) in chunks:
        q8a.attn_accumulate_chunk(st, q, kp + s * row, vp + s * row, kv_dtype, s, n, N * row,
                                  H * N * row, causal)
        if on_state is not None:
            torch.cuda.synchronize()
            on_state(s, n, m, l, o)
    if not finalize:
        return None, None, (m, l, o)
    out = torch.empty((B, H, M, D), dtype=torch.float16, device=dev())
    lse = torch.empty((B, H, M), dtype=torch.float32, device=dev())
    q8a.attn_finalize(st, out, lse)
    torch.cuda.synchronize()
    return out, lse, (m, l, o)


def metrics(out_rows: np.ndarray, lse_rows: np.ndarray, O_ref: np.ndarray,
            lse_ref: np.ndarray):
    o = out_rows.astype(np.float64)
    err = np.abs(o - O_ref)
    max_abs = float(err.max()) if err.size else 0.0
    rel_rms = float(np.sqrt((err ** 2).sum() / max((O_ref ** 2).sum(), 1e-300)))
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse_rows), fin), "LSE finiteness differs"
    lse_err = float((np.abs(lse_rows[fin].astype(np.float64) - lse_ref[fin]) /
                     np.maximum(1.0, np.abs(lse_ref[fin]))).max()) if fin.any() else 0.0
    return max_abs, rel_rms, lse_err


def assert_close(out_rows, lse_rows, O_ref, lse_ref, label=""):
    max_abs, rel_rms, lse_err = metrics(out_rows, lse_rows, O_ref, lse_ref)
    say("%s max-abs %.3e rel-rms %.3e lse-rel %.3e" % (label, max_abs, rel_rms, lse_err))
    assert max_abs <= MAX_ABS, (label, max_abs)
    assert rel_rms <= REL_RMS, (label, rel_rms)
    assert lse_err <= LSE_REL, (label, lse_err)
    return max_abs, rel_rms, lse_err


def rows_of(t: torch.Tensor, rows: np.ndarray, last=None):
    """Pick flat rows (b*H + h)*M + i of a [B, H, M(, 64)] device tensor, as numpy."""
    a = t.detach().cpu()
    if last:
        a = a.reshape(-1, last)
    else:
        a = a.reshape(-1)
    if a.dtype == torch.float16:
        a = a.float()
    return a.numpy()[rows]
