// Chunked causal attention over a Q8_0 (or FP16) KV cache: state init, the fused per-chunk
// accumulate kernel and finalize.
//
// The method is the chunk recurrence of "Out-of-Core Flash Streaming & Speculative Decode
// (1M Context)", Sec. 3 ("Chunked FlashAttention: Exact Mathematical Derivation"): per query row
// the state (m, l, O) survives between chunk calls in device memory; a chunk updates it with
// S = Q K^T / sqrt(D), m' = max(m, max_j S_j), alpha = e^(m - m'), beta_j = e^(S_j - m'),
// l' = l alpha + sum beta, O' = O alpha + sum beta_j V_j.  Keys and values are block_q8_0
// ("Core Architecture & The 4-Brick Pipeline", Sec. 5).
//
// Accumulate kernel, one workgroup = 4 wavefronts = 128 query rows of one (sequence, head):
//   * K/V tiles of 64 keys are fetched with 128-bit buffer loads (out-of-range bytes read as 0)
//     into LDS as raw Q8_0 rows, then unpacked in LDS:
//       - K: the exact int8 values times the FP16 scale, split into two FP16 halves
//         hi = fp16(q*d) and lo = q*d - hi (exact, q*d has at most 18 significant bits), so
//         Q.K^T on FP16 MFMA reproduces the dequantised logits up to FP32 accumulation;
//       - V: the exact int8 values as FP16, transposed to [dim][key]; its FP16 scales are kept
//         per key and folded into the probabilities (P * d16, FP16) before the PV product.
//   * Each wavefront owns 32 query rows and computes S^T = K Q^T with v_mfma_f32_32x32x16_f16,
//     so each lane holds 16 logits of ONE query: the row max needs one cross-lane step and the
//     rescale factor is per lane.  P stays in registers as the B operand of O^T += V^T P^T; the
//     key order of the transposed V tile is permuted to match the accumulator layout.
//   * Softmax in base 2 with 1/sqrt(64)*log2(e) folded into one FMA.  The reference maximum is
//     raised only when a tile's maximum exceeds it by more than 8 (log2 units), so O and l are
//     rarely rescaled; the state written back is renormalised to the true running maximum.
//   * Tiles wholly above the causal diagonal are skipped ("Core Architecture ...", Sec. 5,
//     causal skipping); rows that see no key of the chunk are not written.
//   * A state row whose m is -inf is empty: its O and l are not read.
#include <hip/hip_fp16.h>

#include "q8attn_internal.h"

namespace q8a {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int QT = 128;  // query rows per workgroup
constexpr int WQ = 32;   // query rows per wavefront
constexpr int KT = 64;   // keys per LDS tile
constexpr int NTHR = 256;
constexpr int KP = 72;   // LDS pitch (halves) of the K tiles (144-byte rows)
constexpr int VP = 72;   // LDS pitch (halves) of the transposed V tile
constexpr float kScaleLog2 = 0.125f * 1.44269504088896340736f; // 1/sqrt(64) * log2(e)
constexpr float kTau = 8.0f; // lazy rescale threshold, log2 units

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, bytes, 0x00020000);
}

// 16 bytes at byte offset `off` of a buffer whose size is `bytes` (a multiple of 4).  Bytes past
// the end read as zero; a 16-byte piece that straddles the end is fetched as four dwords so that
// the in-range dwords are kept.
__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t bytes)
{
    if (off + 16u <= bytes || off >= bytes)
        return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    u32x4 x;
    x[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    x[1] = __builtin_amdgcn_raw_buffer_load_b32(r, off + 4, 0, 0);
    x[2] = __builtin_amdgcn_raw_buffer_load_b32(r, off + 8, 0, 0);
    x[3] = __builtin_amdgcn_raw_buffer_load_b32(r, off + 12, 0, 0);
    return x;
}

// Four signed bytes -> four FP16 values (exact).  Each byte is biased to unsigned, placed in the
// mantissa of 1024.0 (0x6400), and 1024 + 128 is subtracted.
__device__ __forceinline__ void i8x4_to_f16(uint32_t w, half2v &lo, half2v &hi)
{
    const uint32_t u = w ^ 0x80808080u;
    const uint32_t a = (u & 0xffu) | ((u & 0xff00u) << 8) | 0x64006400u;
    const uint32_t b = ((u >> 16) & 0xffu) | ((u >> 8) & 0xff0000u) | 0x64006400u;
    const half2v bias = {(_Float16)1152.0f, (_Float16)1152.0f};
    lo = __builtin_bit_cast(half2v, a) - bias;
    hi = __builtin_bit_cast(half2v, b) - bias;
}

__device__ __forceinline__ uint32_t byte_of(uint32_t x, int i) { return (x >> (8 * i)) & 0xffu; }

// Position of key r (0..63) inside the transposed V tile and the V-scale vector: bits 2 and 3
// swapped, so that the 8 keys one lane contributes to a PV step are contiguous.
__device__ __forceinline__ int vpos(int r)
{
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

__device__ __forceinline__ half8 to_half8(const floatx16 &s, int base)
{
    half8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        r[j] = (_Float16)s[base + j];
    return r;
}

template <int FMT> // 0: Q8_0 rows (68 bytes), 1: FP16 rows (128 bytes)
__global__ __launch_bounds__(NTHR) void accumulate_kernel(AccumulateArgs a)
{
    constexpr int ROW = FMT == 0 ? kQ8RowBytes : kF16RowBytes;
    constexpr int RAW = KT * ROW;
    constexpr int RAW16 = RAW / 16;
    __shared__ __align__(16) uint8_t raw[2][RAW];
    __shared__ __align__(16) _Float16 khi[KT * KP];
    __shared__ __align__(16) _Float16 klo[FMT == 0 ? KT * KP : 8];
    __shared__ __align__(16) _Float16 vt[64 * VP];
    __shared__ __align__(16) _Float16 vsc[FMT == 0 ? 2 * KT : 8];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int qcol = lane & 31, g = lane >> 5;
    const int qt = (int)gridDim.x - 1 - (int)blockIdx.x; // tiles with more visible keys first
    const int h = blockIdx.y, b = blockIdx.z;
    const int64_t head = (int64_t)b * a.H + h;

    // keys [0, end) of the chunk are visible to query row qrow
    auto kv_end_for = [&](int qrow) -> int {
        if (!a.causal)
            return a.n_kv;
        const int64_t e = a.q_pos0 + qrow - a.kv_pos0 + 1;
        return (int)(e < 0 ? 0 : (e > a.n_kv ? a.n_kv : e));
    };
    const int q_wg0 = qt * QT;
    const int kv_end_wg = kv_end_for(min(q_wg0 + QT, a.M) - 1);
    if (kv_end_wg <= 0)
        return; // the whole workgroup sees nothing of this chunk
    const int n_tiles = (kv_end_wg + KT - 1) / KT;

    const int q_w0 = q_wg0 + wave * WQ;
    const bool wave_live = q_w0 < a.M;
    const bool wave_full = q_w0 + WQ <= a.M;
    const int kv_end_w = wave_live ? kv_end_for(min(q_w0 + WQ, a.M) - 1) : 0;
    const int kv_full_w = wave_full ? kv_end_for(q_w0) : 0; // visible to every row of the wave
    const bool active = kv_end_w > 0;

    const int qi = q_w0 + qcol;
    const bool q_ok = qi < a.M;
    const int64_t qpos = a.q_pos0 + qi;
    const int64_t row = head * a.M + qi;

    half8 qreg[4];
    floatx16 o0, o1;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        o0[v] = 0.f;
        o1[v] = 0.f;
    }
    float l_part = 0.f;
    float m_raw = -INFINITY; // running max of the raw dot products Q.K (scaled logit * 8)
    float m_ref = -INFINITY; // reference maximum of the exponentials, log2 units
    bool saw = false;
    if (active && q_ok) {
        const half8 *qrow = reinterpret_cast<const half8 *>(
            reinterpret_cast<const _Float16 *>(a.q) + row * kHeadDim);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            qreg[kk] = qrow[2 * kk + g];
        const float mo = a.m[row];
        if (mo != -INFINITY) {
            m_raw = mo * 8.0f;
            m_ref = m_raw * kScaleLog2;
            if (g == 0)
                l_part = a.l[row];
            const float4 *orow = reinterpret_cast<const float4 *>(a.o + row * kHeadDim);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float4 x = orow[2 * k + g];
                const float4 y = orow[8 + 2 * k + g];
                o0[4 * k + 0] = x.x; o0[4 * k + 1] = x.y; o0[4 * k + 2] = x.z; o0[4 * k + 3] = x.w;
                o1[4 * k + 0] = y.x; o1[4 * k + 1] = y.y; o1[4 * k + 2] = y.z; o1[4 * k + 3] = y.w;
            }
        }
    } else {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            qreg[kk] = half8{};
    }

    const uint8_t *kbase = a.k + b * a.kv_seq_stride + h * a.kv_head_stride;
    const uint8_t *vbase = a.v + b * a.kv_seq_stride + h * a.kv_head_stride;
    const uint32_t head_bytes = (uint32_t)a.n_kv * ROW;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase, head_bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase, head_bytes);

    for (int t = 0; t < n_tiles; ++t) {
        const int key0 = t * KT;
        // ---- 1. raw K and V rows of keys [key0, key0 + 64) -> LDS (coalesced 128-bit loads)
        for (int i = tid; i < RAW16; i += NTHR) {
            const uint32_t off = (uint32_t)key0 * ROW + 16u * i;
            *reinterpret_cast<u32x4 *>(&raw[0][16 * i]) = load16(rk, off, head_bytes);
            *reinterpret_cast<u32x4 *>(&raw[1][16 * i]) = load16(rv, off, head_bytes);
        }
        __syncthreads();

        // ---- 2. unpack into the MFMA operand tiles
        if constexpr (FMT == 0) {
            { // K: thread = (block, key, 16-value half of the block); waves 0-1 block 0, 2-3 block 1
                const int blk = tid >> 7, key = (tid & 127) >> 1, hh = tid & 1;
                const uint8_t *rr = &raw[0][key * 68];
                uint32_t w[4];
                if (blk == 0) { // values at byte 2 + 16*hh: realign by 2 bytes
                    const uint32_t *p = reinterpret_cast<const uint32_t *>(rr + 16 * hh);
                    const uint32_t x0 = p[0], x1 = p[1], x2 = p[2], x3 = p[3], x4 = p[4];
                    w[0] = __builtin_amdgcn_alignbyte(x1, x0, 2);
                    w[1] = __builtin_amdgcn_alignbyte(x2, x1, 2);
                    w[2] = __builtin_amdgcn_alignbyte(x3, x2, 2);
                    w[3] = __builtin_amdgcn_alignbyte(x4, x3, 2);
                } else {        // values at byte 36 + 16*hh: dword aligned
                    const uint32_t *p = reinterpret_cast<const uint32_t *>(rr + 36 + 16 * hh);
                    w[0] = p[0]; w[1] = p[1]; w[2] = p[2]; w[3] = p[3];
                }
                const _Float16 d = *reinterpret_cast<const _Float16 *>(rr + 34 * blk);
                const half2v d2 = {d, d};
                half8 hi8[2], lo8[2];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    half2v q01, q23;
                    i8x4_to_f16(w[i], q01, q23);
                    const half2v h01 = q01 * d2, h23 = q23 * d2;
                    const half2v l01 = __builtin_elementwise_fma(q01, d2, -h01);
                    const half2v l23 = __builtin_elementwise_fma(q23, d2, -h23);
                    hi8[i >> 1][4 * (i & 1) + 0] = h01[0]; hi8[i >> 1][4 * (i & 1) + 1] = h01[1];
                    hi8[i >> 1][4 * (i & 1) + 2] = h23[0]; hi8[i >> 1][4 * (i & 1) + 3] = h23[1];
                    lo8[i >> 1][4 * (i & 1) + 0] = l01[0]; lo8[i >> 1][4 * (i & 1) + 1] = l01[1];
                    lo8[i >> 1][4 * (i & 1) + 2] = l23[0]; lo8[i >> 1][4 * (i & 1) + 3] = l23[1];
                }
                half8 *dh = reinterpret_cast<half8 *>(&khi[key * KP + 32 * blk + 16 * hh]);
                half8 *dl = reinterpret_cast<half8 *>(&klo[key * KP + 32 * blk + 16 * hh]);
                dh[0] = hi8[0]; dh[1] = hi8[1];
                dl[0] = lo8[0]; dl[1] = lo8[1];
            }
            { // V: thread = (4 keys, 4 dims); transposed to [dim][vpos(key)]
                const int kq = tid & 15, dg = tid >> 4, blk = dg >> 3;
                uint32_t x[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint8_t *rr = &raw[1][(4 * kq + c) * 68];
                    if (blk == 0) {
                        const uint32_t *p = reinterpret_cast<const uint32_t *>(rr + 4 * dg);
                        x[c] = __builtin_amdgcn_alignbyte(p[1], p[0], 2);
                    } else {
                        x[c] = *reinterpret_cast<const uint32_t *>(rr + 36 + 4 * (dg - 8));
                    }
                }
                const int p0 = vpos(4 * kq);
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const uint32_t y = byte_of(x[0], d) | (byte_of(x[1], d) << 8) |
                                       (byte_of(x[2], d) << 16) | (byte_of(x[3], d) << 24);
                    half2v lo, hi;
                    i8x4_to_f16(y, lo, hi);
                    const half4 r4 = {lo[0], lo[1], hi[0], hi[1]};
                    *reinterpret_cast<half4 *>(&vt[(4 * dg + d) * VP + p0]) = r4;
                }
                if (tid < 2 * KT) {
                    const int key = tid & 63, sb = tid >> 6;
                    vsc[sb * KT + vpos(key)] =
                        *reinterpret_cast<const _Float16 *>(&raw[1][key * 68 + 34 * sb]);
                }
            }
        } else {
            { // K: straight copy into the padded tile
                const int key = tid >> 2, qq = tid & 3;
                const u32x4 *src = reinterpret_cast<const u32x4 *>(&raw[0][key * 128 + 32 * qq]);
                u32x4 *dst = reinterpret_cast<u32x4 *>(&khi[key * KP + 16 * qq]);
                dst[0] = src[0];
                dst[1] = src[1];
            }
            { // V: thread = (4 keys, 4 dims); transposed to [dim][vpos(key)]
                const int kq = tid & 15, dg = tid >> 4;
                half4 x[4];
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    x[c] = *reinterpret_cast<const half4 *>(&raw[1][(4 * kq + c) * 128 + 8 * dg]);
                const int p0 = vpos(4 * kq);
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const half4 r4 = {x[0][d], x[1][d], x[2][d], x[3][d]};
                    *reinterpret_cast<half4 *>(&vt[(4 * dg + d) * VP + p0]) = r4;
                }
            }
        }
        __syncthreads();

        // ---- 3. this wavefront's 32 query rows against the 64 keys of the tile
        if (key0 < kv_end_w) {
            floatx16 s[2];
#pragma unroll
            for (int sub = 0; sub < 2; ++sub) {
                floatx16 acc;
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    acc[v] = 0.f;
                const int kr = (32 * sub + qcol) * KP + 8 * g;
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const half8 ah = *reinterpret_cast<const half8 *>(&khi[kr + 16 * kk]);
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, qreg[kk], acc, 0, 0, 0);
                    if constexpr (FMT == 0) {
                        const half8 al = *reinterpret_cast<const half8 *>(&klo[kr + 16 * kk]);
                        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, qreg[kk], acc, 0, 0, 0);
                    }
                }
                s[sub] = acc;
            }
            // lane (qcol, g) holds S^T[key 32*sub + 8*(v/4) + 4*g + v%4][query qcol]
            if (key0 + KT > kv_full_w) {
#pragma unroll
                for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int kc = key0 + 32 * sub + 8 * (v >> 2) + 4 * g + (v & 3);
                        const bool ok = q_ok && kc < a.n_kv &&
                                        (!a.causal || a.kv_pos0 + kc <= qpos);
                        s[sub][v] = ok ? s[sub][v] : -INFINITY;
                    }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int v = 0; v < 16; ++v)
                mx = fmaxf(mx, fmaxf(s[0][v], s[1][v]));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            m_raw = fmaxf(m_raw, mx);
            saw = saw || (mx != -INFINITY);
            const float mx2 = mx * kScaleLog2;
            const bool need = mx2 > m_ref + kTau;
            if (__builtin_amdgcn_ballot_w64(need)) {
                const float m_new = need ? mx2 : m_ref;
                const float alpha =
                    (m_ref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_new);
                l_part *= alpha;
                o0 *= alpha;
                o1 *= alpha;
                m_ref = m_new;
            }
            const float base = (m_ref == -INFINITY) ? 0.f : m_ref;
            float lsum = 0.f;
#pragma unroll
            for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sub][v], kScaleLog2, -base));
                    s[sub][v] = p;
                    lsum += p;
                }
            l_part += lsum;
#pragma unroll
            for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    const half8 p16 = to_half8(s[sub], 8 * tt);
                    const int pos = 32 * sub + 16 * tt + 8 * g;
                    half8 b0, b1;
                    if constexpr (FMT == 0) {
                        b0 = p16 * *reinterpret_cast<const half8 *>(&vsc[pos]);
                        b1 = p16 * *reinterpret_cast<const half8 *>(&vsc[KT + pos]);
                    } else {
                        b0 = p16;
                        b1 = p16;
                    }
                    const half8 a0 = *reinterpret_cast<const half8 *>(&vt[qcol * VP + pos]);
                    const half8 a1 = *reinterpret_cast<const half8 *>(&vt[(32 + qcol) * VP + pos]);
                    o0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b0, o0, 0, 0, 0);
                    o1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b1, o1, 0, 0, 0);
                }
        }
    }

    // ---- write back the rows that saw at least one key, renormalised to the true maximum
    if (active) {
        const float l_tot = l_part + __shfl_xor(l_part, 32);
        if (q_ok && saw) {
            const float r = __builtin_amdgcn_exp2f(m_ref - m_raw * kScaleLog2);
            float4 *orow = reinterpret_cast<float4 *>(a.o + row * kHeadDim);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                orow[2 * k + g] = make_float4(o0[4 * k] * r, o0[4 * k + 1] * r,
                                              o0[4 * k + 2] * r, o0[4 * k + 3] * r);
                orow[8 + 2 * k + g] = make_float4(o1[4 * k] * r, o1[4 * k + 1] * r,
                                                  o1[4 * k + 2] * r, o1[4 * k + 3] * r);
            }
            if (g == 0) {
                a.m[row] = m_raw * 0.125f;
                a.l[row] = l_tot * r;
            }
        }
    }
}

__global__ __launch_bounds__(256) void state_init_kernel(float *m, float *l, int64_t n_rows)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n_rows) {
        m[i] = -INFINITY;
        l[i] = 0.f;
    }
}

// out = O / l rounded once to FP16; lse = m + ln l.  Eight lanes per row, 8 values each.
__global__ __launch_bounds__(256) void finalize_kernel(const float *__restrict__ m,
                                                       const float *__restrict__ l,
                                                       const float4 *__restrict__ o,
                                                       half8 *__restrict__ out,
                                                       float *__restrict__ lse, int64_t n_rows)
{
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = gid >> 3;
    const int part = (int)(gid & 7);
    if (row >= n_rows)
        return;
    const float mv = m[row];
    half8 res;
    if (mv == -INFINITY) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            res[j] = (_Float16)0.0f;
        if (part == 0 && lse)
            lse[row] = -INFINITY;
    } else {
        const float lv = l[row];
        const float4 x = o[row * 16 + 2 * part];
        const float4 y = o[row * 16 + 2 * part + 1];
        res[0] = (_Float16)(x.x / lv); res[1] = (_Float16)(x.y / lv);
        res[2] = (_Float16)(x.z / lv); res[3] = (_Float16)(x.w / lv);
        res[4] = (_Float16)(y.x / lv); res[5] = (_Float16)(y.y / lv);
        res[6] = (_Float16)(y.z / lv); res[7] = (_Float16)(y.w / lv);
        if (part == 0 && lse)
            lse[row] = mv + logf(lv);
    }
    out[row * 8 + part] = res;
}

} // namespace

hipError_t launch_state_init(float *m, float *l, int64_t n_rows, hipStream_t s)
{
    const int64_t grid = (n_rows + 255) / 256;
    hipLaunchKernelGGL(state_init_kernel, dim3((unsigned)grid), dim3(256), 0, s, m, l, n_rows);
    return hipGetLastError();
}

hipError_t launch_accumulate(const AccumulateArgs &a, int kv_dtype, hipStream_t s)
{
    const dim3 grid((unsigned)((a.M + QT - 1) / QT), (unsigned)a.H, (unsigned)a.B);
    if (kv_dtype == 0)
        hipLaunchKernelGGL(accumulate_kernel<0>, grid, dim3(NTHR), 0, s, a);
    else
        hipLaunchKernelGGL(accumulate_kernel<1>, grid, dim3(NTHR), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_finalize(const float *m, const float *l, const float *o, void *out,
                           float *lse, int64_t n_rows, hipStream_t s)
{
    const int64_t grid = (n_rows * 8 + 255) / 256;
    hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)grid), dim3(256), 0, s, m, l,
                       reinterpret_cast<const float4 *>(o), reinterpret_cast<half8 *>(out), lse,
                       n_rows);
    return hipGetLastError();
}

} // namespace q8a
