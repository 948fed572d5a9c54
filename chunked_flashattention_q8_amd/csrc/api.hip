// C ABI of libq8attn.so: argument validation, launch configuration and the double-buffered
// host-to-device streaming loop.  Every check runs before anything is enqueued; on failure the
// state descriptor is left as it was.
#include <errno.h>
#include <stdint.h>
#include <unistd.h>

#include <thread>

#include "q8attn.h"
#include "q8attn_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

int hip_failure(hipError_t e)
{
    g_last_hip_error = (int)e;
    return Q8A_E_HIP;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// query rows per (sequence, head): a head's O rows (256 bytes each) are addressed with 32-bit
// byte offsets
constexpr int32_t kMaxRows = (1 << 24) - 1;

int row_bytes(int32_t kv_dtype)
{
    return kv_dtype == Q8A_KV_Q8_0 ? q8a::kQ8RowBytes
                                   : (kv_dtype == Q8A_KV_F16 ? q8a::kF16RowBytes : 0);
}

int check_state(const q8a_state *st)
{
    if (!st || st->magic != Q8A_STATE_MAGIC || (st->flags & ~Q8A_STATE_FLAGS_KNOWN) ||
        (st->flags & Q8A_FORM_MASK) > Q8A_FORM_SPLIT)
        return Q8A_E_STATE;
    if (st->head_dim != q8a::kHeadDim || st->n_seq < 1 || st->n_heads < 1 || st->n_q < 1 ||
        !st->m || !st->l || !st->o || st->q_pos0 < 0)
        return Q8A_E_STATE;
    // sizes attn_state_init refuses as unsupported (a descriptor edited by hand): the launch
    // geometry relies on them
    if (st->n_heads > 65535 || st->n_seq > 65535 || st->n_q > kMaxRows ||
        (int64_t)st->n_seq * st->n_heads > ((int64_t)1 << 23) ||
        (int64_t)st->n_seq * st->n_heads * st->n_q > ((int64_t)1 << 28))
        return Q8A_E_UNSUPPORTED;
    return Q8A_OK;
}

int64_t state_rows(const q8a_state *st)
{
    return (int64_t)st->n_seq * st->n_heads * st->n_q;
}

// Validation shared by the resident and the streamed accumulate paths.
int check_chunk(const q8a_state *st, const void *q, const void *k, const void *v,
                int32_t kv_dtype, int64_t kv_pos0, int32_t n_kv, int64_t head_stride,
                int64_t seq_stride, int32_t causal)
{
    int rc = check_state(st);
    if (rc)
        return rc;
    const int row = row_bytes(kv_dtype);
    if (!row)
        return Q8A_E_INVAL;
    if (!q || !k || !v || n_kv < 1 || kv_pos0 < 0 || (causal != 0 && causal != 1))
        return Q8A_E_INVAL;
    if ((int64_t)n_kv * row > INT32_MAX - 16) // per-head byte range is addressed with 32 bits
        return Q8A_E_INVAL;
    if (kv_pos0 > INT64_MAX / 2 || st->q_pos0 > INT64_MAX / 2)
        return Q8A_E_INVAL;
    if (head_stride < 0 || seq_stride < 0)
        return Q8A_E_INVAL;
    if (st->n_heads > 1 && head_stride < (int64_t)n_kv * row)
        return Q8A_E_INVAL;
    if (st->n_seq > 1 && seq_stride < (int64_t)n_kv * row)
        return Q8A_E_INVAL;
    if (st->n_heads > 65535 || st->n_seq > 65535 || st->n_q > kMaxRows)
        return Q8A_E_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || head_stride % 16 ||
        seq_stride % 16)
        return Q8A_E_ALIGN;
    return Q8A_OK;
}

q8a::AccumulateArgs make_args(const q8a_state *st, const void *q, const void *k, const void *v,
                              int64_t kv_pos0, int32_t n_kv, int64_t head_stride,
                              int64_t seq_stride, int32_t causal)
{
    q8a::AccumulateArgs a;
    a.q = q;
    a.k = static_cast<const uint8_t *>(k);
    a.v = static_cast<const uint8_t *>(v);
    a.m = st->m;
    a.l = st->l;
    a.o = st->o;
    a.kv_head_stride = head_stride;
    a.kv_seq_stride = seq_stride;
    a.q_pos0 = st->q_pos0;
    a.kv_pos0 = kv_pos0;
    a.B = st->n_seq;
    a.H = st->n_heads;
    a.M = st->n_q;
    a.n_kv = n_kv;
    a.causal = causal;
    a.out = nullptr;
    a.lse = nullptr;
    a.final_out_only = 0;
    a.fresh = 0;
    switch (st->flags & Q8A_FORM_MASK) {
    case Q8A_FORM_WIDE: a.form = q8a::kFormWide; break;
    case Q8A_FORM_NARROW: a.form = q8a::kFormNarrow; break;
    case Q8A_FORM_KEY_SPLIT: a.form = q8a::kFormKeySplit; break;
    case Q8A_FORM_SPLIT: a.form = q8a::kFormSplit; break;
    default: a.form = q8a::kFormAuto;
    }
    return a;
}

// A state described by attn_state_init_deferred (Q8A_STATE_FRESH) holds nothing yet.  Before the
// launch of a chunk that every query row sees, the kernel itself treats every row as empty and
// writes it (a.fresh); otherwise the initialisation is enqueued here first.
hipError_t prepare_fresh(const q8a_state *st, q8a::AccumulateArgs &a, hipStream_t s)
{
    if (!(st->flags & Q8A_STATE_FRESH))
        return hipSuccess;
    if (!a.causal || st->q_pos0 >= a.kv_pos0) {
        a.fresh = 1;
        return hipSuccess;
    }
    return q8a::launch_state_init(st->m, st->l, state_rows(st), s);
}

// Before a call that reads the state as it stands (finalize, merge): initialise a fresh state.
hipError_t settle_fresh(q8a_state *st, hipStream_t s)
{
    if (!(st->flags & Q8A_STATE_FRESH))
        return hipSuccess;
    hipError_t e = q8a::launch_state_init(st->m, st->l, state_rows(st), s);
    if (e == hipSuccess)
        st->flags &= ~Q8A_STATE_FRESH;
    return e;
}

// Enqueue one accumulate launch (plus the initialisation a fresh state may still owe); clears
// Q8A_STATE_FRESH once enqueued.
hipError_t accumulate(q8a_state *st, q8a::AccumulateArgs &a, int kv_dtype, hipStream_t s)
{
    hipError_t e = prepare_fresh(st, a, s);
    if (e == hipSuccess)
        e = q8a::launch_accumulate(a, kv_dtype, s);
    if (e == hipSuccess)
        st->flags &= ~Q8A_STATE_FRESH;
    return e;
}

// The arguments of attn_state_init and attn_state_init_deferred.
int check_init(q8a_state *st, float *m, float *l, float *o, int32_t n_seq, int32_t n_heads,
               int32_t n_q, int32_t head_dim, int64_t q_pos0)
{
    if (!st || !m || !l || !o || n_seq < 1 || n_heads < 1 || n_q < 1 || q_pos0 < 0)
        return Q8A_E_INVAL;
    if (head_dim != q8a::kHeadDim)
        return Q8A_E_UNSUPPORTED;
    // launches stay below 2^32 work-items: 8 lanes per state row in finalize and merge, one
    // 256-thread workgroup per 256 rows of each (sequence, head) in accumulate
    if (n_heads > 65535 || n_seq > 65535 || n_q > kMaxRows ||
        (int64_t)n_seq * n_heads > ((int64_t)1 << 23) ||
        (int64_t)n_seq * n_heads * n_q > ((int64_t)1 << 28))
        return Q8A_E_UNSUPPORTED;
    if (!aligned(m, 4) || !aligned(l, 4) || !aligned(o, 16))
        return Q8A_E_ALIGN;
    return Q8A_OK;
}

void describe(q8a_state *st, float *m, float *l, float *o, int32_t n_seq, int32_t n_heads,
              int32_t n_q, int32_t head_dim, int64_t q_pos0, uint32_t flags)
{
    st->m = m;
    st->l = l;
    st->o = o;
    st->n_seq = n_seq;
    st->n_heads = n_heads;
    st->n_q = n_q;
    st->head_dim = head_dim;
    st->q_pos0 = q_pos0;
    st->magic = Q8A_STATE_MAGIC;
    st->flags = flags;
}

} // namespace

extern "C" {

const char *q8a_status_string(int status)
{
    switch (status) {
    case Q8A_OK: return "ok";
    case Q8A_E_INVAL: return "invalid argument";
    case Q8A_E_UNSUPPORTED: return "unsupported configuration";
    case Q8A_E_ALIGN: return "misaligned pointer or stride";
    case Q8A_E_STATE: return "state descriptor not initialised or inconsistent";
    case Q8A_E_HIP: return "HIP runtime error";
    case Q8A_E_IO: return "file read failed or file too short";
    default: return "unknown status";
    }
}

int q8a_last_hip_error(void) { return g_last_hip_error; }

int q8_0_pack(const float *x, void *dst, int64_t n_rows, int32_t row_len, void *stream)
{
    if (n_rows < 0 || row_len <= 0 || row_len % 32)
        return Q8A_E_INVAL;
    if (n_rows == 0)
        return Q8A_OK;
    if (!x || !dst)
        return Q8A_E_INVAL;
    if (n_rows > ((int64_t)1 << 28) / (row_len / 32)) // 8 lanes per block: < 2^32 work-items
        return Q8A_E_INVAL;
    if (!aligned(x, 16) || !aligned(dst, 2))
        return Q8A_E_ALIGN;
    const int64_t n_blocks = n_rows * (row_len / 32);
    hipError_t e = q8a::launch_q8_0_pack(x, static_cast<uint8_t *>(dst), n_blocks,
                                          static_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q8A_OK : hip_failure(e);
}

int attn_state_init(q8a_state *st, float *m, float *l, float *o, int32_t n_seq,
                    int32_t n_heads, int32_t n_q, int32_t head_dim, int64_t q_pos0,
                    void *stream)
{
    int rc = check_init(st, m, l, o, n_seq, n_heads, n_q, head_dim, q_pos0);
    if (rc)
        return rc;
    const int64_t rows = (int64_t)n_seq * n_heads * n_q;
    hipError_t e = q8a::launch_state_init(m, l, rows, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_failure(e);
    describe(st, m, l, o, n_seq, n_heads, n_q, head_dim, q_pos0, 0);
    return Q8A_OK;
}

int attn_state_init_deferred(q8a_state *st, float *m, float *l, float *o, int32_t n_seq,
                             int32_t n_heads, int32_t n_q, int32_t head_dim, int64_t q_pos0)
{
    int rc = check_init(st, m, l, o, n_seq, n_heads, n_q, head_dim, q_pos0);
    if (rc)
        return rc;
    describe(st, m, l, o, n_seq, n_heads, n_q, head_dim, q_pos0, Q8A_STATE_FRESH);
    return Q8A_OK;
}

int attn_accumulate_chunk(q8a_state *st, const void *q, const void *k, const void *v,
                          int32_t kv_dtype, int64_t kv_pos0, int32_t n_kv,
                          int64_t kv_head_stride, int64_t kv_seq_stride, int32_t causal,
                          void *stream)
{
    int rc = check_chunk(st, q, k, v, kv_dtype, kv_pos0, n_kv, kv_head_stride, kv_seq_stride,
                         causal);
    if (rc)
        return rc;
    q8a::AccumulateArgs a =
        make_args(st, q, k, v, kv_pos0, n_kv, kv_head_stride, kv_seq_stride, causal);
    hipError_t e = accumulate(st, a, kv_dtype, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q8A_OK : hip_failure(e);
}

int attn_accumulate_chunk_final(q8a_state *st, const void *q, const void *k,
                                const void *v, int32_t kv_dtype, int64_t kv_pos0, int32_t n_kv,
                                int64_t kv_head_stride, int64_t kv_seq_stride, int32_t causal,
                                void *out, float *lse, void *stream)
{
    int rc = check_chunk(st, q, k, v, kv_dtype, kv_pos0, n_kv, kv_head_stride, kv_seq_stride,
                         causal);
    if (rc)
        return rc;
    if (causal != 1 || !out)
        return Q8A_E_INVAL;
    if (!aligned(out, 16) || (lse && !aligned(lse, 4)))
        return Q8A_E_ALIGN;
    // the outputs must not overlap anything the launch reads or writes
    const int64_t rows = state_rows(st);
    auto overlap = [](const void *a, int64_t na, const void *b, int64_t nb) {
        const char *x = static_cast<const char *>(a), *y = static_cast<const char *>(b);
        return x < y + nb && y < x + na;
    };
    const int64_t row = kv_dtype == Q8A_KV_Q8_0 ? q8a::kQ8RowBytes : q8a::kF16RowBytes;
    const int64_t kv_span = (int64_t)(st->n_seq - 1) * kv_seq_stride +
                            (int64_t)(st->n_heads - 1) * kv_head_stride + (int64_t)n_kv * row;
    const void *used[6] = {q, k, v, st->m, st->l, st->o};
    const int64_t spans[6] = {rows * q8a::kHeadDim * 2, kv_span, kv_span, rows * 4, rows * 4,
                              rows * q8a::kHeadDim * 4};
    for (int i = 0; i < 6; ++i)
        if (overlap(out, rows * q8a::kHeadDim * 2, used[i], spans[i]) ||
            (lse && overlap(lse, rows * 4, used[i], spans[i])))
            return Q8A_E_INVAL;
    if (lse && overlap(out, rows * q8a::kHeadDim * 2, lse, rows * 4))
        return Q8A_E_INVAL;
    q8a::AccumulateArgs a =
        make_args(st, q, k, v, kv_pos0, n_kv, kv_head_stride, kv_seq_stride, causal);
    a.out = out;
    a.lse = lse;
    a.final_out_only = (st->flags & Q8A_STATE_FINAL_OUT_ONLY) ? 1 : 0;
    hipError_t e = accumulate(st, a, kv_dtype, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q8A_OK : hip_failure(e);
}

int attn_append_chunk(q8a_state *st, const void *q, const float *k_new,
                      const float *v_new, void *k_cache, void *v_cache, int64_t kv_pos0,
                      int32_t n_kv, int64_t kv_head_stride, int64_t kv_seq_stride,
                      int32_t causal, void *stream)
{
    int rc = check_chunk(st, q, k_cache, v_cache, Q8A_KV_Q8_0, kv_pos0, n_kv, kv_head_stride,
                         kv_seq_stride, causal);
    if (rc)
        return rc;
    if (!k_new || !v_new)
        return Q8A_E_INVAL;
    if (!aligned(k_new, 16) || !aligned(v_new, 16))
        return Q8A_E_ALIGN;
    const int64_t runs = (int64_t)st->n_seq * st->n_heads;
    if (runs > 65535)
        return Q8A_E_UNSUPPORTED;
    if (kv_head_stride > ((int64_t)1 << 46) || kv_seq_stride > ((int64_t)1 << 46))
        return Q8A_E_INVAL; // keeps the span products below in range
    const int64_t row_span = (int64_t)n_kv * q8a::kQ8RowBytes;
    // every (sequence, head) destination run must be its own: sequences outside heads or heads
    // outside sequences (check_chunk covers the single-sequence and single-head cases)
    if (st->n_seq > 1 && st->n_heads > 1 &&
        !(kv_seq_stride >= (st->n_heads - 1) * kv_head_stride + row_span ||
          kv_head_stride >= (st->n_seq - 1) * kv_seq_stride + row_span))
        return Q8A_E_INVAL;
    // K and V destinations must not overlap each other or the sources
    const int64_t dst_span = (int64_t)(st->n_seq - 1) * kv_seq_stride +
                             (int64_t)(st->n_heads - 1) * kv_head_stride + row_span;
    const int64_t src_span = runs * n_kv * q8a::kHeadDim * 4;
    auto overlap = [](const void *a, int64_t na, const void *b, int64_t nb) {
        const char *x = static_cast<const char *>(a), *y = static_cast<const char *>(b);
        return x < y + nb && y < x + na;
    };
    // ... nor Q or the state, which the accumulate reads after the pack has written
    const int64_t rows = state_rows(st);
    const void *reads[5] = {k_new, v_new, q, st->m, st->l};
    const int64_t spans[5] = {src_span, src_span, rows * q8a::kHeadDim * 2, rows * 4, rows * 4};
    if (overlap(k_cache, dst_span, v_cache, dst_span) ||
        overlap(k_cache, dst_span, st->o, rows * q8a::kHeadDim * 4) ||
        overlap(v_cache, dst_span, st->o, rows * q8a::kHeadDim * 4))
        return Q8A_E_INVAL;
    for (int i = 0; i < 5; ++i)
        if (overlap(k_cache, dst_span, reads[i], spans[i]) ||
            overlap(v_cache, dst_span, reads[i], spans[i]))
            return Q8A_E_INVAL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = q8a::launch_q8_0_pack_rows(k_new, v_new, static_cast<uint8_t *>(k_cache),
                                              static_cast<uint8_t *>(v_cache), st->n_seq,
                                              st->n_heads, n_kv, kv_head_stride, kv_seq_stride,
                                              s);
    if (e != hipSuccess)
        return hip_failure(e);
    q8a::AccumulateArgs a = make_args(st, q, k_cache, v_cache, kv_pos0, n_kv, kv_head_stride,
                                      kv_seq_stride, causal);
    e = accumulate(st, a, Q8A_KV_Q8_0, s);
    return e == hipSuccess ? Q8A_OK : hip_failure(e);
}

int attn_finalize(q8a_state *st, void *out, float *lse, void *stream)
{
    int rc = check_state(st);
    if (rc)
        return rc;
    if (!out)
        return Q8A_E_INVAL;
    if (!aligned(out, 16) || (lse && !aligned(lse, 4)))
        return Q8A_E_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = settle_fresh(st, s);
    if (e == hipSuccess)
        e = q8a::launch_finalize(st->m, st->l, st->o, out, lse, state_rows(st), s);
    return e == hipSuccess ? Q8A_OK : hip_failure(e);
}

int attn_state_merge(q8a_state *dst, const q8a_state *src, void *stream)
{
    int rc = check_state(dst);
    if (rc)
        return rc;
    rc = check_state(src);
    if (rc)
        return rc;
    if (dst->n_seq != src->n_seq || dst->n_heads != src->n_heads || dst->n_q != src->n_q ||
        dst->q_pos0 != src->q_pos0)
        return Q8A_E_STATE;
    const int64_t rows = state_rows(dst);
    // the two states must not share memory (a state merged with itself would count its keys
    // twice; overlapping buffers would race)
    auto overlap = [](const void *a, int64_t na, const void *b, int64_t nb) {
        const char *x = static_cast<const char *>(a), *y = static_cast<const char *>(b);
        return x < y + nb && y < x + na;
    };
    const float *dm[3] = {dst->m, dst->l, dst->o}, *sm[3] = {src->m, src->l, src->o};
    const int64_t bytes[3] = {rows * 4, rows * 4, rows * 4 * q8a::kHeadDim};
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j)
            if (overlap(dm[i], bytes[i], sm[j], bytes[j]))
                return Q8A_E_INVAL;
    if (src->flags & Q8A_STATE_FRESH)
        return Q8A_OK; // src holds no key: nothing to merge
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = settle_fresh(dst, s);
    if (e == hipSuccess)
        e = q8a::launch_merge(dst->m, dst->l, dst->o, src->m, src->l, src->o, rows, s);
    return e == hipSuccess ? Q8A_OK : hip_failure(e);
}

int attn_accumulate_stream(q8a_state *st, const void *q, const void *k_host,
                           const void *v_host, int32_t kv_dtype, int64_t n_kv_total,
                           int32_t chunk_tokens, void *const slot_k[2], void *const slot_v[2],
                           int32_t causal, void *compute_stream, void *copy_stream)
{
    if (!slot_k || !slot_v || !k_host || !v_host || n_kv_total < 1 || chunk_tokens < 1)
        return Q8A_E_INVAL;
    for (int s = 0; s < 2; ++s)
        if (!slot_k[s] || !slot_v[s])
            return Q8A_E_INVAL;
    if (st && st->magic == Q8A_STATE_MAGIC && n_kv_total > INT64_MAX / 4)
        return Q8A_E_INVAL;
    const int row = row_bytes(kv_dtype);
    const int64_t head_stride = (int64_t)chunk_tokens * row;
    int rc = check_chunk(st, q, slot_k[0], slot_v[0], kv_dtype, 0, chunk_tokens, head_stride,
                         head_stride * (st ? st->n_heads : 1), causal);
    if (rc)
        return rc;
    for (int s = 1; s < 2; ++s)
        if (!aligned(slot_k[s], 16) || !aligned(slot_v[s], 16))
            return Q8A_E_ALIGN;
    const int64_t seq_stride = head_stride * st->n_heads;
    const int64_t chunk_bytes = seq_stride * st->n_seq;
    const int64_t n_chunks = (n_kv_total + chunk_tokens - 1) / chunk_tokens;
    hipStream_t cs = static_cast<hipStream_t>(compute_stream);
    hipStream_t ds = static_cast<hipStream_t>(copy_stream);
    const uint8_t *kh = static_cast<const uint8_t *>(k_host);
    const uint8_t *vh = static_cast<const uint8_t *>(v_host);

    hipEvent_t ev_full[2] = {nullptr, nullptr}, ev_free[2] = {nullptr, nullptr};
    hipEvent_t ev_start = nullptr;
    hipError_t e = hipSuccess;
    auto destroy = [&]() {
        for (int s = 0; s < 2; ++s) {
            if (ev_full[s]) (void)hipEventDestroy(ev_full[s]);
            if (ev_free[s]) (void)hipEventDestroy(ev_free[s]);
        }
        if (ev_start) (void)hipEventDestroy(ev_start);
    };
    for (int s = 0; s < 2 && e == hipSuccess; ++s) {
        e = hipEventCreateWithFlags(&ev_full[s], hipEventDisableTiming);
        if (e == hipSuccess)
            e = hipEventCreateWithFlags(&ev_free[s], hipEventDisableTiming);
    }
    if (e == hipSuccess)
        e = hipEventCreateWithFlags(&ev_start, hipEventDisableTiming);
    // the slots may still be read by earlier work on the compute stream
    if (e == hipSuccess)
        e = hipEventRecord(ev_start, cs);
    if (e == hipSuccess)
        e = hipStreamWaitEvent(ds, ev_start, 0);
    for (int64_t c = 0; c < n_chunks && e == hipSuccess; ++c) {
        const int s = (int)(c & 1);
        const int64_t kv_pos0 = c * chunk_tokens;
        const int32_t n_kv = (int32_t)((n_kv_total - kv_pos0) < chunk_tokens
                                           ? (n_kv_total - kv_pos0) : chunk_tokens);
        if (c >= 2)
            e = hipStreamWaitEvent(ds, ev_free[s], 0); // chunk c-2 has finished with slot s
        if (e == hipSuccess)
            e = hipMemcpyAsync(slot_k[s], kh + c * chunk_bytes, (size_t)chunk_bytes,
                               hipMemcpyHostToDevice, ds);
        if (e == hipSuccess)
            e = hipMemcpyAsync(slot_v[s], vh + c * chunk_bytes, (size_t)chunk_bytes,
                               hipMemcpyHostToDevice, ds);
        if (e == hipSuccess)
            e = hipEventRecord(ev_full[s], ds);
        if (e == hipSuccess)
            e = hipStreamWaitEvent(cs, ev_full[s], 0);
        if (e == hipSuccess) {
            q8a::AccumulateArgs a = make_args(st, q, slot_k[s], slot_v[s], kv_pos0, n_kv,
                                              head_stride, seq_stride, causal);
            e = accumulate(st, a, kv_dtype, cs);
        }
        if (e == hipSuccess)
            e = hipEventRecord(ev_free[s], cs);
    }
    destroy();
    return e == hipSuccess ? Q8A_OK : hip_failure(e);
}

} // extern "C"

namespace {

// The 4096-byte-aligned range covering [off, off + len): pread over it (O_DIRECT needs aligned
// offsets, sizes and buffers); the file may end inside the rounded tail, not before off + len.
bool read_aligned(int fd, uint8_t *buf, int64_t off, int64_t len)
{
    const int64_t a0 = off & ~(int64_t)4095;
    const int64_t want = ((off + len + 4095) & ~(int64_t)4095) - a0;
    const int64_t need = off + len - a0;
    int64_t got = 0;
    while (got < need) {
        const ssize_t r = pread(fd, buf + got, (size_t)(want - got), (off_t)(a0 + got));
        if (r < 0) {
            if (errno == EINTR)
                continue;
            return false;
        }
        if (r == 0)
            break; // end of file
        got += r;
    }
    return got >= need;
}

} // namespace

int attn_accumulate_file(q8a_state *st, const void *q, int fd_k, int fd_v,
                         int64_t file_offset, int32_t kv_dtype, int64_t n_kv_total,
                         int32_t chunk_tokens, void *const ring_k[2], void *const ring_v[2],
                         int64_t ring_bytes, void *const slot_k[2], void *const slot_v[2],
                         int32_t causal, void *compute_stream, void *copy_stream)
{
    if (!slot_k || !slot_v || !ring_k || !ring_v || n_kv_total < 1 || chunk_tokens < 1 ||
        fd_k < 0 || fd_v < 0 || file_offset < 0)
        return Q8A_E_INVAL;
    for (int s = 0; s < 2; ++s)
        if (!slot_k[s] || !slot_v[s] || !ring_k[s] || !ring_v[s])
            return Q8A_E_INVAL;
    if (st && st->magic == Q8A_STATE_MAGIC && n_kv_total > INT64_MAX / 4)
        return Q8A_E_INVAL;
    const int row = row_bytes(kv_dtype);
    const int64_t head_stride = (int64_t)chunk_tokens * row;
    int rc = check_chunk(st, q, slot_k[0], slot_v[0], kv_dtype, 0, chunk_tokens, head_stride,
                         head_stride * (st ? st->n_heads : 1), causal);
    if (rc)
        return rc;
    for (int s = 0; s < 2; ++s) {
        if (!aligned(slot_k[s], 16) || !aligned(slot_v[s], 16))
            return Q8A_E_ALIGN;
        if (!aligned(ring_k[s], 4096) || !aligned(ring_v[s], 4096))
            return Q8A_E_ALIGN;
    }
    const int64_t seq_stride = head_stride * st->n_heads;
    const int64_t chunk_bytes = seq_stride * st->n_seq;
    if (ring_bytes < chunk_bytes + 8192)
        return Q8A_E_INVAL;
    const int64_t n_chunks = (n_kv_total + chunk_tokens - 1) / chunk_tokens;
    if (file_offset > INT64_MAX / 2 || n_chunks > (INT64_MAX / 2) / chunk_bytes)
        return Q8A_E_INVAL;
    hipStream_t cs = static_cast<hipStream_t>(compute_stream);
    hipStream_t ds = static_cast<hipStream_t>(copy_stream);

    hipEvent_t ev_full[2] = {nullptr, nullptr}, ev_free[2] = {nullptr, nullptr};
    hipEvent_t ev_start = nullptr;
    hipError_t e = hipSuccess;
    int status = Q8A_OK;
    auto destroy = [&]() {
        for (int s = 0; s < 2; ++s) {
            if (ev_full[s]) (void)hipEventDestroy(ev_full[s]);
            if (ev_free[s]) (void)hipEventDestroy(ev_free[s]);
        }
        if (ev_start) (void)hipEventDestroy(ev_start);
    };
    for (int s = 0; s < 2 && e == hipSuccess; ++s) {
        e = hipEventCreateWithFlags(&ev_full[s], hipEventDisableTiming);
        if (e == hipSuccess)
            e = hipEventCreateWithFlags(&ev_free[s], hipEventDisableTiming);
    }
    if (e == hipSuccess)
        e = hipEventCreateWithFlags(&ev_start, hipEventDisableTiming);
    // the slots may still be read by earlier work on the compute stream
    if (e == hipSuccess)
        e = hipEventRecord(ev_start, cs);
    if (e == hipSuccess)
        e = hipStreamWaitEvent(ds, ev_start, 0);
    // chunk c of both files into ring slot s: K on this thread, V on a second one (or here
    // too, should a thread not start)
    auto read_chunk = [&](int64_t c, int s) -> bool {
        const int64_t off = file_offset + c * chunk_bytes;
        bool ok_v = false;
        auto read_v = [&] {
            ok_v = read_aligned(fd_v, static_cast<uint8_t *>(ring_v[s]), off, chunk_bytes);
        };
        std::thread tv;
        try {
            tv = std::thread(read_v);
        } catch (...) {
            read_v();
        }
        const bool ok_k = read_aligned(fd_k, static_cast<uint8_t *>(ring_k[s]), off,
                                       chunk_bytes);
        if (tv.joinable())
            tv.join();
        return ok_k && ok_v;
    };
    if (e == hipSuccess && !read_chunk(0, 0))
        status = Q8A_E_IO;
    for (int64_t c = 0; c < n_chunks && e == hipSuccess && status == Q8A_OK; ++c) {
        const int s = (int)(c & 1);
        const int64_t kv_pos0 = c * chunk_tokens;
        const int32_t n_kv = (int32_t)((n_kv_total - kv_pos0) < chunk_tokens
                                           ? (n_kv_total - kv_pos0) : chunk_tokens);
        // chunk c+1 is read into the other slot while chunk c is copied and accumulated; that
        // slot was last copied from for chunk c-1, whose copies must have completed
        const bool has_next = c + 1 < n_chunks;
        bool next_ok = true;
        std::thread reader;
        if (has_next) {
            if (c >= 1)
                e = hipEventSynchronize(ev_full[s ^ 1]);
            if (e != hipSuccess)
                break;
            try {
                reader = std::thread([&, c, s] { next_ok = read_chunk(c + 1, s ^ 1); });
            } catch (...) {
                next_ok = read_chunk(c + 1, s ^ 1); // no overlap, same result
            }
        }
        const int64_t delta = (file_offset + c * chunk_bytes) & 4095;
        const uint8_t *rk = static_cast<const uint8_t *>(ring_k[s]);
        const uint8_t *rv = static_cast<const uint8_t *>(ring_v[s]);
        if (c >= 2)
            e = hipStreamWaitEvent(ds, ev_free[s], 0); // chunk c-2 has finished with slot s
        if (e == hipSuccess)
            e = hipMemcpyAsync(slot_k[s], rk + delta, (size_t)chunk_bytes,
                               hipMemcpyHostToDevice, ds);
        if (e == hipSuccess)
            e = hipMemcpyAsync(slot_v[s], rv + delta, (size_t)chunk_bytes,
                               hipMemcpyHostToDevice, ds);
        if (e == hipSuccess)
            e = hipEventRecord(ev_full[s], ds);
        if (e == hipSuccess)
            e = hipStreamWaitEvent(cs, ev_full[s], 0);
        if (e == hipSuccess) {
            q8a::AccumulateArgs a = make_args(st, q, slot_k[s], slot_v[s], kv_pos0, n_kv,
                                              head_stride, seq_stride, causal);
            e = accumulate(st, a, kv_dtype, cs);
        }
        if (e == hipSuccess)
            e = hipEventRecord(ev_free[s], cs);
        if (reader.joinable())
            reader.join();
        if (!next_ok)
            status = Q8A_E_IO;
    }
    // the ring buffers are free once their last copies have completed
    for (int s = 0; s < 2 && e == hipSuccess && n_chunks > s; ++s)
        e = hipEventSynchronize(ev_full[s]);
    destroy();
    if (e != hipSuccess)
        return hip_failure(e);
    return status;
}
