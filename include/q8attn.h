/*
 * q8attn.h -- exact chunked causal attention prefill over a Q8_0 KV cache, for AMD MI355X (gfx950).
 *
 * The method ("Out-of-Core Flash Streaming & Speculative Decode (1M Context)", m4-prefill-engine,
 * Sec. 3 "Chunked FlashAttention: Exact Mathematical Derivation"): the KV sequence arrives in
 * chunks; for every query row i the running state (m_i, l_i, O_i) -- the largest scaled logit seen
 * so far, the sum of e^(S_ij - m_i), and the unnormalised output sum of e^(S_ij - m_i) V_j -- is
 * kept in device memory between chunk calls and updated with the rescale factor
 * e^(m_old - m_new), so that O/l after the last chunk equals single-pass softmax(QK^T/sqrt(D)) V.
 * Keys and values are stored as Q8_0 ("Core Architecture & The 4-Brick Pipeline", Sec. 5,
 * block_q8_0): blocks of 32 values, each an FP16 scale followed by 32 int8, 34 bytes; a 64-dim
 * head row is two blocks, 68 bytes.
 *
 * Conventions shared by every call
 *   - Pointers are DEVICE pointers unless the name ends in _host.  The caller owns every buffer
 *     and every stream and keeps buffers alive until the enqueued work has completed.
 *   - Every call is asynchronous on `stream` (a hipStream_t passed as void*; NULL = the legacy
 *     default stream).  No call allocates or frees device memory or synchronises the host.
 *   - All argument checks run on the host before anything is enqueued; on failure nothing is
 *     launched and the state descriptor is unchanged.  A failing HIP runtime call (for example
 *     no device) returns Q8A_E_HIP and its hipError_t is kept for q8a_last_hip_error().  Faults
 *     inside kernels surface at the caller's next synchronisation.
 *   - head_dim must be 64.  Layouts are head-major: Q and the output [B][H][M][64] FP16,
 *     state m and l [B][H][M] FP32, state O [B][H][M][64] FP32.  Query row i of every sequence
 *     sits at absolute position q_pos0 + i; chunk key j at absolute position kv_pos0 + j.
 *   - Causal rule: a query at position p sees the keys at positions <= p (diagonal included).
 *   - Supported value range: finite inputs with |x| < 30000 for K and V (larger Q8_0 scales can
 *     overflow FP16 intermediates); scores are computed in FP32.
 */
#ifndef Q8ATTN_H
#define Q8ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    Q8A_OK = 0,
    Q8A_E_INVAL = 1,       /* bad pointer, size, position or enum value */
    Q8A_E_UNSUPPORTED = 2, /* a valid request this library does not implement (e.g. head_dim) */
    Q8A_E_ALIGN = 3,       /* a pointer or stride breaks the stated alignment */
    Q8A_E_STATE = 4,       /* descriptor not initialised, or it does not match the call */
    Q8A_E_HIP = 5,         /* a HIP runtime call failed; see q8a_last_hip_error() */
    Q8A_E_IO = 6           /* a file read failed or the file ended early (attn_accumulate_file) */
} q8a_status;

typedef enum {
    Q8A_KV_Q8_0 = 0, /* K and V rows of 68 bytes: [fp16 d0][32 x int8][fp16 d1][32 x int8] */
    Q8A_KV_F16 = 1   /* K and V rows of 64 FP16 values (128 bytes) */
} q8a_kv_dtype;

#define Q8A_STATE_MAGIC 0x51384154u /* "Q8AT" */

/* Host-side descriptor of a caller-owned online-softmax state.  Filled by attn_state_init (or
 * attn_state_init_deferred); the other calls only read it, except that they clear
 * Q8A_STATE_FRESH.  A state row whose m is -inf is EMPTY: it has seen no key, its l is 0 and its
 * O is treated as zero and never read (so O need not be cleared).
 * A descriptor of sequences [s0, s0 + n) of an initialised state is a copy of its descriptor
 * with m and l advanced by s0*n_heads*n_q floats, o by 64 times that, and n_seq = n; it may be
 * passed wherever a state is (for example to merge sequence blocks of one state).  Take such
 * copies only of a descriptor without Q8A_STATE_FRESH (each copy would initialise on its own).
 * Every call that reads a descriptor checks it as attn_state_init checks its arguments: a
 * descriptor edited to sizes that call refuses gives Q8A_E_UNSUPPORTED, one without the magic,
 * with head_dim other than 64 or with unknown flag bits Q8A_E_STATE. */
typedef struct {
    float *m;          /* [n_seq][n_heads][n_q]      running maximum of the scaled logits  */
    float *l;          /* [n_seq][n_heads][n_q]      running sum of e^(S - m)             */
    float *o;          /* [n_seq][n_heads][n_q][64]  running sum of e^(S - m) V           */
    int32_t n_seq, n_heads, n_q, head_dim;
    int64_t q_pos0;    /* absolute position of query row 0 (same for every sequence) */
    uint32_t magic;    /* Q8A_STATE_MAGIC once initialised */
    uint32_t flags;    /* Q8A_STATE_* and Q8A_FORM_* bits below; other bits must be 0 */
} q8a_state;

/* Bits of q8a_state.flags.
 *
 * Q8A_STATE_FRESH: the device buffers hold nothing yet.  Set by attn_state_init_deferred, which
 *   enqueues no work; the first call that reads the state then treats every row as empty and
 *   writes it.  An accumulate call (any attn_accumulate_* or attn_append_chunk) whose first
 *   chunk is seen by every query row (causal = 0, or q_pos0 >= the chunk's kv_pos0; for the
 *   streamed calls the first chunk starts at position 0) writes every row itself in that
 *   chunk's launch and reads nothing of the old state; any other call first enqueues the same
 *   initialisation attn_state_init does.  The call clears the bit in the caller's descriptor
 *   once that work is enqueued; on an error return before it the bit is left set.  A merge
 *   with a FRESH src has nothing to merge and enqueues nothing.
 * Q8A_STATE_FINAL_OUT_ONLY: attn_accumulate_chunk_final writes the out and lse of the rows a
 *   call completes and NOT their m, l and O, which keep what they held before the call (a
 *   completed row of a causal pass in ascending key order sees no later key, so its state is
 *   dead).  Everything else, and every other call, is unchanged.  After such a pass, the
 *   completed rows' state must not be finalised, merged or accumulated further.
 * Q8A_FORM_*: the accumulate kernel's tile form for states of more than 64 query rows, for
 *   tuning and tests (Q8A_FORM_AUTO, 0, lets the library choose; see attn_accumulate_chunk).
 *   WIDE and NARROW give the same results bit for bit; KEY_SPLIT and SPLIT sum in other orders
 *   and agree with them to rounding.  Values above Q8A_FORM_SPLIT are reserved (Q8A_E_STATE). */
#define Q8A_STATE_FRESH 0x1u
#define Q8A_STATE_FINAL_OUT_ONLY 0x2u
#define Q8A_FORM_MASK 0x70u
#define Q8A_FORM_AUTO 0x00u      /* the library's choice */
#define Q8A_FORM_WIDE 0x10u      /* 256 query rows per workgroup, 4 wavefronts */
#define Q8A_FORM_NARROW 0x20u    /* 128 query rows per workgroup, 4 wavefronts */
#define Q8A_FORM_KEY_SPLIT 0x30u /* 256 query rows, 8 wavefronts splitting each tile's keys */
#define Q8A_FORM_SPLIT 0x40u     /* 64 query rows, 4 wavefronts splitting each tile's keys */
#define Q8A_STATE_FLAGS_KNOWN (Q8A_STATE_FRESH | Q8A_STATE_FINAL_OUT_ONLY | Q8A_FORM_MASK)

/* Q8_0 pack ("Core Architecture & The 4-Brick Pipeline", Sec. 5, block_q8_0; row size from
 * "Out-of-Core Flash Streaming ...", Sec. 1).
 *   x       FP32 [n_rows][row_len], C-contiguous, 16-byte aligned.
 *   dst     n_rows * row_len/32 * 34 bytes, 2-byte aligned; block k of the flat sequence at byte
 *           34*k: the FP16 scale (little-endian) then 32 int8.
 *   row_len positive multiple of 32 (64 for a KV head row); n_rows >= 0 (0 enqueues nothing);
 *           at most 2^28 blocks per call (else Q8A_E_INVAL).
 * Per block: amax = max|x|, d = amax/127 (FP32, correctly rounded), d16 = FP16(d) (round to
 * nearest even), q = round(x / d16) (FP32 division, halves away from zero), clamped to
 * [-127, 127]; an all-zero block stores d16 = 0 and q = 0.  Bit-exact with the CPU oracle. */
int q8_0_pack(const float *x, void *dst, int64_t n_rows, int32_t row_len, void *stream);

/* Describe a state and make every row empty: writes m = -inf and l = 0 for all
 * n_seq*n_heads*n_q rows (O is not written; see q8a_state).
 *   m, l    FP32 [n_seq][n_heads][n_q], 4-byte aligned;  o  FP32 [...][64], 16-byte aligned.
 *   head_dim must be 64 (else Q8A_E_UNSUPPORTED); n_seq, n_heads, n_q >= 1; q_pos0 >= 0.
 *   n_seq, n_heads <= 65535, n_q <= 16,777,215 (a head's O rows are addressed with 32-bit byte
 *   offsets), n_seq*n_heads <= 2^23 and n_seq*n_heads*n_q <= 2^28 (every launch stays below 2^32
 *   work-items), else Q8A_E_UNSUPPORTED. */
int attn_state_init(q8a_state *st, float *m, float *l, float *o, int32_t n_seq,
                    int32_t n_heads, int32_t n_q, int32_t head_dim, int64_t q_pos0,
                    void *stream);

/* attn_state_init with the device writes deferred: checks the same arguments and fills the same
 * descriptor, with flags = Q8A_STATE_FRESH, and enqueues nothing (no stream argument).  The
 * first call on the state initialises the rows (see Q8A_STATE_FRESH); a causal prefill whose
 * first chunk starts at or before the first query position (as in a prefill from key 0) then
 * needs no initialisation launch at all.  The initial state is the one of "Out-of-Core ...",
 * Sec. 3 before its first chunk: every row empty (m = -inf, l = 0). */
int attn_state_init_deferred(q8a_state *st, float *m, float *l, float *o, int32_t n_seq,
                             int32_t n_heads, int32_t n_q, int32_t head_dim, int64_t q_pos0);

/* Accumulate one KV chunk into the state (the recurrence of "Out-of-Core Flash Streaming ...",
 * Sec. 3, steps 1-6).
 *   q        FP16 [n_seq][n_heads][n_q][64], 16-byte aligned (same Q on every call).
 *   k, v     address of key 0 of the chunk for sequence 0, head 0.  Key j of (seq b, head h) is
 *            at  k + b*kv_seq_stride + h*kv_head_stride + j*row  (row = 68 bytes for Q8_0,
 *            128 for FP16).  16-byte aligned; both strides are byte counts, multiples of 16,
 *            and at least n_kv*row.  Reads are 16-byte pieces: when n_kv*row is not a multiple
 *            of 16, up to 12 bytes after a head's last key are read (never past the 16-byte
 *            block holding that key's last byte) and ignored.
 *   kv_pos0  absolute position of chunk key 0 (>= 0);  n_kv  chunk length, >= 1 (a partial
 *            last chunk is fine).
 *   causal   1: the triangular mask of Mode A ("Out-of-Core ...", Sec. 4); 0: every chunk key
 *            is visible to every query.
 * A row that sees no key of the chunk is left bit-for-bit untouched (tiles that lie wholly above
 * the diagonal are skipped, as in "Core Architecture ...", Sec. 5).  Workgroups take 256 query
 * rows unless n_seq*n_heads*ceil(n_q/256) would not fill the device's workgroup slots (two per
 * compute unit): then 128 rows when, with the causal mask, the first query row sees less than
 * half the chunk keys the last row sees, else, with at most one such workgroup per compute unit,
 * 256 rows whose tile keys are split over 8 wavefronts.  For more than 64 rows the Q8A_FORM_*
 * bits of st->flags fix the form instead.  Each key position must be accumulated exactly once
 * per state; chunk order is free.  Calls on one state must be stream-ordered; calls on different
 * states are independent.  st is written only to clear Q8A_STATE_FRESH. */
int attn_accumulate_chunk(q8a_state *st, const void *q, const void *k, const void *v,
                          int32_t kv_dtype, int64_t kv_pos0, int32_t n_kv,
                          int64_t kv_head_stride, int64_t kv_seq_stride, int32_t causal,
                          void *stream);

/* attn_accumulate_chunk, and in the same launch the final output of the rows this chunk
 * completes ("Out-of-Core ...", Sec. 3: the final normalisation O / l and m + ln l, applied as
 * soon as a row has seen its last key).  With causal masking and the chunks of a pass given in
 * ascending key order, a row whose query position p lies inside the chunk (kv_pos0 <= p <
 * kv_pos0 + n_kv) sees no key of any later chunk: its out and lse are written as attn_finalize
 * would write them from the state after this call, bit for bit.  Other rows' out and lse are
 * not touched, and the state is updated exactly as by attn_accumulate_chunk (so attn_finalize
 * still works afterwards) -- unless st->flags holds Q8A_STATE_FINAL_OUT_ONLY: then the completed
 * rows' m, l and O are not written (their state is dead in such a pass).  The caller guarantees
 * the order: every key before kv_pos0 that such a row sees must already be in the state.
 *   causal   must be 1 (Q8A_E_INVAL otherwise).
 *   out      FP16 [n_seq][n_heads][n_q][64], 16-byte aligned;  lse  FP32 [..][n_q], 4-byte
 *            aligned, or NULL.  Neither may overlap Q, K, V, the state or each other
 *            (Q8A_E_INVAL).
 * Everything else as for attn_accumulate_chunk. */
int attn_accumulate_chunk_final(q8a_state *st, const void *q, const void *k,
                                const void *v, int32_t kv_dtype, int64_t kv_pos0, int32_t n_kv,
                                int64_t kv_head_stride, int64_t kv_seq_stride, int32_t causal,
                                void *out, float *lse, void *stream);

/* Quantise-on-append: pack n_kv newly appended tokens of K and V into the Q8_0 cache and
 * accumulate them into the state, in one call.  The cache entries are quantised dynamically as
 * they arrive ("Core Architecture & The 4-Brick Pipeline", Sec. 5: dynamically quantised
 * block_q8_0 KV; the append of Mode A in "Out-of-Core ...", Sec. 4).  The result is exactly that of
 * q8_0_pack of each new row into its cache row followed by attn_accumulate_chunk over those rows:
 * the same cache bytes, the same state bits.
 *   k_new, v_new   FP32 [n_seq][n_heads][n_kv][64], C-contiguous, 16-byte aligned (device).
 *   k_cache, v_cache  destination of new key 0 for sequence 0, head 0; key j of (seq b, head h)
 *            goes to  k_cache + b*kv_seq_stride + h*kv_head_stride + j*68.  Same alignment, stride
 *            and over-read rules as attn_accumulate_chunk with kv_dtype Q8_0; strides at most
 *            2^46 bytes.  With several sequences and several heads, the (sequence, head) runs must
 *            not interleave: kv_seq_stride >= (n_heads-1)*kv_head_stride + n_kv*68, or the same
 *            with the roles swapped.  The K and V destinations must not overlap each other or
 *            the FP32 sources, Q or the state (Q8A_E_INVAL).  Only the n_kv*68 bytes of each run
 *            are written; should the accumulate launch fail (Q8A_E_HIP), the cache rows are
 *            written and the state is not.
 *   q, kv_pos0, n_kv, causal, stream: as for attn_accumulate_chunk.
 * Two launches on the stream (one pack of both tensors, one accumulate). */
int attn_append_chunk(q8a_state *st, const void *q, const float *k_new,
                      const float *v_new, void *k_cache, void *v_cache, int64_t kv_pos0,
                      int32_t n_kv, int64_t kv_head_stride, int64_t kv_seq_stride,
                      int32_t causal, void *stream);

/* Final output after the last chunk ("Out-of-Core ...", Sec. 3): out = O / l in FP16, formed as
 * O times the correctly rounded FP32 reciprocal of l, in FP32, rounded once to FP16 (nearest
 * even; before that rounding within 1.5 FP32 ulps of O / l), and lse = m + ln(l) in FP32
 * (natural log).  Empty rows give out = 0 and
 * lse = -inf.  out: FP16 [n_seq][n_heads][n_q][64], 16-byte aligned; lse: FP32 [..][n_q] or NULL.
 * The state is not modified (a Q8A_STATE_FRESH state is first initialised, every row empty). */
int attn_finalize(q8a_state *st, void *out, float *lse, void *stream);

/* Merge the partial state src into dst.  Each must hold, for the same rows, the accumulation of
 * a key set, the two key sets disjoint; afterwards dst holds what accumulating both key sets
 * into one state gives (up to rounding): m = max(m_dst, m_src), and l and O of each side
 * rescaled by e^(m_side - m) and added -- the chunk rescale of "Out-of-Core ...", Sec. 3, with
 * src's (m, l, O) in the chunk's place.  Rows empty in src leave dst untouched; rows empty in
 * dst take src's values.  With it a key range can be split over several states that
 * accumulate concurrently (for example on several streams when few query rows leave the GPU
 * idle, as in Mode B of "Out-of-Core ...", Sec. 4) and merged afterwards; the same rule merges
 * states built on different devices.
 *   dst, src  initialised states with equal n_seq, n_heads, n_q and q_pos0 (else Q8A_E_STATE),
 *             whose buffers do not overlap (else Q8A_E_INVAL).  src is not modified.  A
 *             Q8A_STATE_FRESH src holds no key: nothing is enqueued.  A Q8A_STATE_FRESH dst is
 *             first initialised (every row empty).
 * Both states must be stream-ordered before the call (dst and src work on `stream` or
 * synchronised with it). */
int attn_state_merge(q8a_state *dst, const q8a_state *src, void *stream);

/* Double-buffered streaming of a KV cache held in pinned host memory ("Out-of-Core ...", Sec. 2:
 * two ping-pong slots, chunk c+1 copied while chunk c is computed, handoff by synchronisation
 * objects rather than spinning).  Chunk c of the cache covers key positions
 * [c*chunk_tokens, min((c+1)*chunk_tokens, n_kv_total)); its bytes sit at
 * k_host + c*chunk_bytes, laid out [n_seq][n_heads][chunk_tokens][row] (the last chunk padded),
 * chunk_bytes = n_seq*n_heads*chunk_tokens*row.  slot_k[2], slot_v[2] are device buffers of
 * chunk_bytes each, 16-byte aligned.  Copies run on copy_stream (hipMemcpyAsync host->device),
 * kernels on compute_stream; HIP events order slot reuse.  On return everything is enqueued;
 * compute_stream carries the completion of the last chunk.  Key positions start at 0. */
int attn_accumulate_stream(q8a_state *st, const void *q, const void *k_host,
                           const void *v_host, int32_t kv_dtype, int64_t n_kv_total,
                           int32_t chunk_tokens, void *const slot_k[2], void *const slot_v[2],
                           int32_t causal, void *compute_stream, void *copy_stream);

/* Out-of-core feed from storage ("Out-of-Core Flash Streaming ...", Sec. 2: KV chunks read from
 * flash with the page cache bypassed into a two-slot ring, then consumed by the GPU): the same
 * work as attn_accumulate_stream, with the chunk-major K and V read from files.
 *   fd_k, fd_v   open file descriptors (the caller opens them, with O_DIRECT to bypass the page
 *                cache); each holds the layout attn_accumulate_stream takes from host memory,
 *                [chunk][n_seq][n_heads][chunk_tokens][row], starting at byte file_offset
 *                (>= 0), the last chunk padded to full size or ending the file.
 *   ring_k, ring_v  two host buffers each, 4096-byte aligned, ring_bytes long, ring_bytes >=
 *                chunk bytes + 8192: each chunk is read with pread over the 4096-byte-aligned
 *                range that covers it (what O_DIRECT needs), then copied to the device from
 *                inside that range.  With O_DIRECT descriptors the ring must be ordinary
 *                page-aligned memory (an anonymous mmap, for example): direct reads into pinned
 *                (hipHostMalloc) memory fail with EFAULT, and the device copy then stages the
 *                pageable buffer.  With buffered descriptors a pinned ring gives asynchronous
 *                copies.
 *   slot_k, slot_v, q, kv_dtype, n_kv_total, chunk_tokens, causal, streams: as for
 *                attn_accumulate_stream.
 * The call blocks the host: chunk c+1 is read while chunk c is copied (copy_stream) and
 * accumulated (compute_stream); a ring buffer is refilled only after its previous copy has
 * completed.  On return every chunk has been read and its work enqueued, and the ring buffers
 * are no longer in use; compute_stream carries the completion of the last chunk.
 * Q8A_E_IO: a read failed or a file ended early; the chunks before it have been accumulated
 * (their work is enqueued), so the state then holds a prefix of the keys. */
int attn_accumulate_file(q8a_state *st, const void *q, int fd_k, int fd_v,
                         int64_t file_offset, int32_t kv_dtype, int64_t n_kv_total,
                         int32_t chunk_tokens, void *const ring_k[2], void *const ring_v[2],
                         int64_t ring_bytes, void *const slot_k[2], void *const slot_v[2],
                         int32_t causal, void *compute_stream, void *copy_stream);

/* Human-readable name of a q8a_status value. */
const char *q8a_status_string(int status);

/* hipError_t of the most recent Q8A_E_HIP returned on the calling thread (0 if none). */
int q8a_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* Q8ATTN_H */
