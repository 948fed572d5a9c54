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
// Accumulate kernel, one workgroup = 4 wavefronts = 256 query rows of one (sequence, head):
//   * K/V tiles of 64 keys are copied as raw rows straight from HBM into LDS two tiles ahead
//     (128-bit buffer loads that write LDS directly; bytes past the chunk read as 0), then
//     unpacked in LDS into a double-buffered operand tile (one barrier per tile):
//       - K: the int8 values q as FP16 (exact), plus two FP32 factors per key built from its
//         block scales d0, d1: the MFMAs over dims 0-31 give S0 = Q.q0, the accumulator is
//         multiplied by d0/d1, the MFMAs over dims 32-63 add S1 = Q.q1, and one FMA with
//         d1*log2(e)/8 yields the base-2 exponent -- the dequantised logit d0 S0 + d1 S1 up to
//         FP32 rounding, with no FP16 rounding of the dequantised K;
//       - V: fp16(q*d), transposed to [dim][key] (one rounding of the dequantised value).
//   * Each wavefront owns two 32-row query blocks (w and 7 - w of the tile, which balances the
//     causal diagonal) and computes S^T = K Q^T with v_mfma_f32_32x32x16_f16, so each lane
//     holds 16 logits of ONE query per 32 keys: the row max needs one cross-lane step and the
//     rescale factor is per lane.  P stays in registers as the B operand of O^T += V^T P^T;
//     the key order of the transposed V tile is permuted to match the accumulator layout.
//   * Softmax in base 2 with 1/sqrt(64)*log2(e) folded into one FMA.  The reference maximum is
//     raised only when a tile's maximum exceeds it by more than 8 (log2 units), so O and l are
//     rarely rescaled; the state written back is renormalised to the true running maximum.
//   * Tiles wholly above the causal diagonal are skipped ("Core Architecture ...", Sec. 5,
//     causal skipping); rows that see no key of the chunk are not written.
//   * A state row whose m is -inf is empty: its O and l are not read.  The first two tiles'
//     copies, Q and m are all in flight together (tile 1's copies still in flight while tile 0
//     is unpacked); l and O of resumed rows are loaded right before the first tile and arrive
//     behind its QK products.  The state rows are written
//     back through LDS, four whole rows per store instruction.
//   * Workgroups are ordered so that each XCD works on a contiguous set of heads (their K/V
//     stay in that XCD's L2) and the query tiles that see the most keys start first.
//   * Up to 64 query rows per (sequence, head) (Mode B, decode-like calls): the split-key form,
//     where the wavefronts split every tile's keys instead of its rows (see SPLIT below).
//   * Launches whose 256-row workgroups would not fill two slots per compute unit (one
//     sequence of 32 heads): 128-row workgroups, one block per wavefront, where the causal
//     diagonal makes the chunk uneven (see NARROW below), else 8-wavefront workgroups that
//     split every tile's keys (see KEY SPLIT below).
//   * The wavefronts' lower blocks stop seeing keys before their upper blocks on the diagonal;
//     from then on a tile runs for the upper block alone.  The state and final rows are stored
//     through the L2 (system scope), not left dirty in it.
#include <hip/hip_fp16.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "q8attn_internal.h"

namespace q8a {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int QT = 256;  // query rows per workgroup (4 wavefronts x 2 blocks of 32)
constexpr int WQ = 32;   // query rows per MFMA block
constexpr int KT = 64;   // keys per LDS tile
constexpr int NTHR = 256;
// tile forms of the accumulate kernel (its FORM argument); see the kernel
constexpr int kWide = 0;     // 256 rows, 4 wavefronts, blocks w and 7 - w over all keys
constexpr int kSplit = 1;    // up to 64 rows, 4 wavefronts, block w & 1 over key half w >> 1
constexpr int kNarrow = 2;   // 128 rows, 4 wavefronts, block w over all keys
constexpr int kKeySplit = 3; // 256 rows, 8 wavefronts, blocks w & 3 and 7 - (w & 3) over key
                             // half w >> 2
constexpr int KP = 72;   // LDS pitch (halves) of the K tiles (144-byte rows)
constexpr int VP = 72;   // LDS pitch (halves) of the transposed V tile
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.693147180559945309417f;
constexpr float kScaleLog2 = 0.125f * kLog2e; // 1/sqrt(64) * log2(e)
constexpr float kTau = 8.0f; // lazy rescale threshold, log2 units
// cache policy of the write-back's buffer stores: sc0 | sc1 (system scope), written through the
// XCD's L2 instead of left dirty in it, so the end-of-launch L2 write-back before the next call
// has less to do (the next call reads the rows from the memory-side cache either way)
constexpr int kStoreThrough = 1 | 16;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, bytes, 0x00020000);
}

// 16 bytes at byte offset `off` of a buffer resource; bytes past its range read as zero.
__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// 16 bytes per lane from a buffer resource straight into LDS: lane l's bytes land at
// lds_base + 16 * l (lds_base wavefront-uniform).  Written as inline assembly so that the
// compiler's automatic waits do not treat every later LDS read as possibly aliasing the copy
// (it cannot tell the copies' destination from the operand tiles, and would wait for each copy
// right after issuing it); the kernel waits for the copies explicitly before its barriers.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(r), "s"(lds_base)
                 : "memory", "m0");
}

// Signed bytes -> FP16 values (exact).  Each byte is biased to unsigned (x ^ 0x80) and placed as
// the low mantissa byte of 1024.0 (0x64 high byte), giving 1024 + 128 + x; subtracting 1152
// leaves x.  v_perm_b32 picks bytes from {S0, S1} (selector 0-3: S1's bytes, 4-7: S0's), so
// with S0 = 0x64646464 one instruction builds two such FP16 values.
constexpr uint32_t kF16Magic = 0x64646464u;
__device__ __forceinline__ half2v biased_pair_to_f16(uint32_t u, uint32_t sel)
{
    const half2v bias = {(_Float16)1152.0f, (_Float16)1152.0f};
    return __builtin_bit_cast(half2v, __builtin_amdgcn_perm(kF16Magic, u, sel)) - bias;
}

// four signed bytes of w -> (bytes 0, 1) and (bytes 2, 3) as FP16 pairs
__device__ __forceinline__ void i8x4_to_f16(uint32_t w, half2v &lo, half2v &hi)
{
    const uint32_t u = w ^ 0x80808080u;
    lo = biased_pair_to_f16(u, 0x04010400u);
    hi = biased_pair_to_f16(u, 0x04030402u);
}

// The same for K values that are kept only when `keep` is 1 and become 0 when it is 0 (the
// products with a block whose scale is 0): (u - 1152) * keep as one fused multiply-add
// u * keep - 1152 * keep, exact for keep = 1, and +0 for keep = 0 (u is finite).
__device__ __forceinline__ void i8x4_to_f16_keep(uint32_t w, half2v keep, half2v nbias,
                                                 half2v &lo, half2v &hi)
{
    const uint32_t u = w ^ 0x80808080u;
    lo = __builtin_elementwise_fma(
        __builtin_bit_cast(half2v, __builtin_amdgcn_perm(kF16Magic, u, 0x04010400u)), keep,
        nbias);
    hi = __builtin_elementwise_fma(
        __builtin_bit_cast(half2v, __builtin_amdgcn_perm(kF16Magic, u, 0x04030402u)), keep,
        nbias);
}

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

__device__ __forceinline__ float vmax3(float a, float b, float c)
{
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// max(x[lane], x[lane ^ 32]): lanes l and l + 32 hold the same query row
__device__ __forceinline__ float half_swap_max(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float half_swap_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The final output out = O / l of a row, formed the same way by the finalize kernel and by the
// accumulate kernel's write-back of the rows a causal chunk completes (so the two agree bit for
// bit): the reciprocal of l correctly rounded (one IEEE division per row), the product with it
// in FP32, then one rounding to FP16 (nearest even).  Before that rounding the value is within
// 1.5 FP32 ulps of O / l.
__device__ __forceinline__ float final_inv_l(float l) { return 1.0f / l; }
__device__ __forceinline__ _Float16 final_out(float o, float rl) { return (_Float16)(o * rl); }

template <int FMT> // 0: Q8_0 rows (68 bytes), 1: FP16 rows (128 bytes)
struct alignas(16) KvTile { // one LDS buffer of unpacked MFMA operands for KT keys
    _Float16 k[KT * KP];                       // K (Q8_0: the int8 values q), [key][dim]
    // Q8_0 logit scales of each key (block scales d0, d1): S = (S0 * kr + S1) * km / kScaleLog2
    // with S0, S1 the products over the two blocks' q; kr = d0 / d1 and km = d1 * kScaleLog2
    // (d1 = 0, where S1 = 0: kr = d0, km = kScaleLog2)
    alignas(16) float kr[FMT == 0 ? KT : 4];
    alignas(16) float km[FMT == 0 ? KT : 4];
    _Float16 vt[64 * VP];                      // V (Q8_0: fp16(q*d)), [dim][vpos]
};

template <int FMT>
struct Smem {
    static constexpr int ROW = FMT == 0 ? kQ8RowBytes : kF16RowBytes;
    uint8_t raw[2][2][KT * ROW]; // [buffer][K, V][raw rows of KT keys]
    KvTile<FMT> tile[2];
};

// Unpack the raw rows of one KV tile (LDS) into MFMA operand layout (LDS), with 256 threads
// (tid 0-255): PART 0 both tensors, 1 K only, 2 V only.
// MASK: Q8_0 keys from valid_keys on get zero scales.  The bytes of a 16-byte piece that runs
// past the chunk end are real memory (see the range rounding in the kernel); when the chunk's
// byte length is a multiple of 16 there is no such piece, every byte past the end reads as 0,
// and those keys unpack to zero scales by themselves.
template <int FMT, bool MASK, int PART = 0>
__device__ __forceinline__ void unpack_tile(const uint8_t *__restrict__ rk,
                                            const uint8_t *__restrict__ rv, KvTile<FMT> &T,
                                            int tid, int valid_keys)
{
    if constexpr (FMT == 0) {
        if constexpr (PART != 2) {
            // K: thread = (key, quarter of the dims); quarter qq = dims 16qq .. 16qq+15, which
            // sit at byte 34*blk + 2 + 16*hh of the row (blk = qq/2, hh = qq%2): read the 5 dwords
            // that cover them and realign (by 2 bytes for block 0, none for block 1).
            const int key = tid >> 2, qq = tid & 3, blk = qq >> 1, hh = qq & 1;
            const uint8_t *rr = rk + key * 68;
            const int off = 34 * blk + 2 + 16 * hh, sh = off & 3;
            const uint32_t *p = reinterpret_cast<const uint32_t *>(rr + (off & ~3));
            const uint32_t x0 = p[0], x1 = p[1], x2 = p[2], x3 = p[3], x4 = p[4];
            const float d0 = (float)*reinterpret_cast<const _Float16 *>(rr);
            const float d1 = (float)*reinterpret_cast<const _Float16 *>(rr + 34);
            // A block whose scale is 0 contributes 0 whatever its int8 values (q * 0).  The
            // second block's products are added unscaled (S0 * kr + S1), so its int8 values are
            // taken as 0 here (in the conversion itself, at no extra instruction); the first
            // block needs nothing, its products are multiplied by kr = d0 / d1 = 0 (or by d0 = 0
            // when both scales are 0).
            uint32_t w[4];
            w[0] = __builtin_amdgcn_alignbyte(x1, x0, sh);
            w[1] = __builtin_amdgcn_alignbyte(x2, x1, sh);
            w[2] = __builtin_amdgcn_alignbyte(x3, x2, sh);
            w[3] = __builtin_amdgcn_alignbyte(x4, x3, sh);
            const bool zero1 = blk == 1 && d1 == 0.f;
            const _Float16 kp = zero1 ? (_Float16)0.0f : (_Float16)1.0f;
            const _Float16 nb = zero1 ? (_Float16)0.0f : (_Float16)-1152.0f;
            const half2v keep = {kp, kp}, nbias = {nb, nb};
            if constexpr (MASK) {
                // (the masked form has no registers to spare for the two factors: a branch)
                if (__builtin_amdgcn_ballot_w64(zero1)) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        w[i] = zero1 ? 0u : w[i];
                }
            }
            half8 q8[2];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                half2v q01, q23;
                if constexpr (MASK)
                    i8x4_to_f16(w[i], q01, q23);
                else
                    i8x4_to_f16_keep(w[i], keep, nbias, q01, q23);
                q8[i >> 1][4 * (i & 1) + 0] = q01[0]; q8[i >> 1][4 * (i & 1) + 1] = q01[1];
                q8[i >> 1][4 * (i & 1) + 2] = q23[0]; q8[i >> 1][4 * (i & 1) + 3] = q23[1];
            }
            half8 *dk = reinterpret_cast<half8 *>(&T.k[key * KP + 16 * qq]);
            dk[0] = q8[0];
            dk[1] = q8[1];
            // the key's two logit scales, computed by its 4 lanes alike (lanes qq = 0, 2 store kr
            // and 1, 3 km, the same values twice: no branch); keys past the chunk end get 0
            // (their raw bytes may be anything; they are masked)
            const float den = d1 != 0.f ? d1 : 1.f;
            // d0 / den: reciprocal, product and one residual correction (within an ulp or so;
            // no branchy IEEE division sequence in the tile loop)
            const float rcp = __builtin_amdgcn_rcpf(den);
            const float r0 = d0 * rcp;
            const float kr = __builtin_fmaf(__builtin_fmaf(-den, r0, d0), rcp, r0);
            const float sc = (qq & 1) ? den * kScaleLog2 : kr;
            ((qq & 1) ? T.km : T.kr)[key] = (!MASK || key < valid_keys) ? sc : 0.f;
        }
        if constexpr (PART != 1) { // V: thread = (4 keys, 4 dims); transposed to [dim][vpos(key)]
            // dims 4*dg .. 4*dg+3 sit at byte 2 + 4*dg + 2*blk of the row (block 1 skips the
            // second scale): realign by 2 bytes for block 0, none for block 1
            const int kq = tid & 15, dg = tid >> 4, blk = dg >> 3;
            const int off = 2 + 4 * dg + 2 * blk, sh = off & 3;
            uint32_t x[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t *p =
                    reinterpret_cast<const uint32_t *>(rv + (4 * kq + c) * 68 + (off & ~3));
                x[c] = __builtin_amdgcn_alignbyte(p[1], p[0], sh);
            }
            // the four keys' scales of this block; keys past the chunk end get 0 (their raw
            // bytes may be anything, and their P is 0)
            _Float16 sc[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const _Float16 d =
                    *reinterpret_cast<const _Float16 *>(rv + (4 * kq + c) * 68 + 34 * blk);
                sc[c] = (!MASK || 4 * kq + c < valid_keys) ? d : (_Float16)0.0f;
            }
            const half2v s01 = {sc[0], sc[1]}, s23 = {sc[2], sc[3]};
            // byte transpose: t01[i] interleaves the bytes of keys 0 and 1 for dims 2i, 2i+1
            // ([k0.d, k1.d, k0.d+1, k1.d+1]), t23[i] those of keys 2 and 3; each FP16 pair
            // (key 0, key 1) or (key 2, key 3) of one dim is then one byte pick.
            const uint32_t u0 = x[0] ^ 0x80808080u, u1 = x[1] ^ 0x80808080u;
            const uint32_t u2 = x[2] ^ 0x80808080u, u3 = x[3] ^ 0x80808080u;
            const uint32_t t01[2] = {__builtin_amdgcn_perm(u1, u0, 0x05010400u),
                                     __builtin_amdgcn_perm(u1, u0, 0x07030602u)};
            const uint32_t t23[2] = {__builtin_amdgcn_perm(u3, u2, 0x05010400u),
                                     __builtin_amdgcn_perm(u3, u2, 0x07030602u)};
            const int p0 = vpos(4 * kq);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t sel = (d & 1) ? 0x04030402u : 0x04010400u;
                // fp16(q * d): one rounding, like P * d in the product's B operand
                const half2v lo = biased_pair_to_f16(t01[d >> 1], sel) * s01;
                const half2v hi = biased_pair_to_f16(t23[d >> 1], sel) * s23;
                const half4 r4 = {lo[0], lo[1], hi[0], hi[1]};
                *reinterpret_cast<half4 *>(&T.vt[(4 * dg + d) * VP + p0]) = r4;
            }
        }
    } else {
        if constexpr (PART != 2) { // K: straight copy into the padded tile
            const int key = tid >> 2, qq = tid & 3;
            const u32x4 *src = reinterpret_cast<const u32x4 *>(rk + key * 128 + 32 * qq);
            u32x4 *dst = reinterpret_cast<u32x4 *>(&T.k[key * KP + 16 * qq]);
            dst[0] = src[0];
            dst[1] = src[1];
        }
        if constexpr (PART != 1) { // V: thread = (4 keys, 4 dims); transposed to [dim][vpos(key)]
            const int kq = tid & 15, dg = tid >> 4;
            half4 x[4];
#pragma unroll
            for (int c = 0; c < 4; ++c)
                x[c] = *reinterpret_cast<const half4 *>(rv + (4 * kq + c) * 128 + 8 * dg);
            const int p0 = vpos(4 * kq);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const half4 r4 = {x[0][d], x[1][d], x[2][d], x[3][d]};
                *reinterpret_cast<half4 *>(&T.vt[(4 * dg + d) * VP + p0]) = r4;
            }
        }
    }
}

// SPLIT (used when a workgroup's query rows fit in 64): instead of two 32-row blocks over all
// keys, wavefront w owns block w & 1 over the keys of subtile w >> 1 (keys 32(w>>1) .. +31 of
// every tile), with an online-softmax state of its own; the two states of a block are merged
// through LDS at the end by the rule attn_state_merge uses.  All four wavefronts then work on
// the 64 rows instead of two of them (each also carrying an empty block).
// NARROW (used when 256-row workgroups would leave compute-unit slots empty, e.g. one sequence
// of 32 heads): a workgroup takes 128 query rows, wavefront w the 32-row block w over all keys,
// so twice as many workgroups share the chip; each K/V tile is unpacked for half as many rows.
// KEY SPLIT (used when 256-row workgroups would leave compute-unit slots empty and every row
// sees the whole chunk, e.g. the cached chunks of one sequence's long context): 8 wavefronts,
// one workgroup per compute unit; wavefronts w and w + 4 own the same two blocks as wavefront w
// of the 256-row form and split every tile's keys (w >> 2: key half), each with a state of its
// own, merged through LDS at the end as in SPLIT.  The SIMDs then run two wavefronts each, and
// each K/V tile is still unpacked once for 256 rows (K by wavefronts 0-3, V by 4-7).
// CLEAN: the chunk's rows end on a 16-byte boundary (n_kv a multiple of 4 for Q8_0, always for
// FP16), so the unpack needs no masking of keys past the chunk end.
template <int FMT, int FORM, bool CLEAN>
__global__ __launch_bounds__(FORM == kKeySplit ? 2 * NTHR : NTHR, FORM == kKeySplit ? 1 : 2)
void accumulate_kernel(AccumulateArgs a)
{
    constexpr bool SPLIT = FORM == kSplit, NARROW = FORM == kNarrow, KS8 = FORM == kKeySplit;
    constexpr bool KSPLIT = SPLIT || KS8;        // wavefronts split every tile's keys
    constexpr int NJ = (SPLIT || NARROW) ? 1 : 2; // 32-row query blocks per wavefront
    constexpr int NS = KSPLIT ? 1 : 2;            // 32-key subtiles per wavefront and tile
    constexpr int QTF = SPLIT ? 2 * WQ : NARROW ? QT / 2 : QT; // query rows per workgroup
    constexpr int ROW = Smem<FMT>::ROW;
    constexpr int RAW16 = KT * ROW / 16;                 // 16-byte pieces per tensor tile
    constexpr int NPRE = KS8 ? 2 : FMT == 0 ? 3 : 4;     // prefetch slots per thread
    // the fewest copies of a tile any thread issues (the prologue's wait counts on them)
    constexpr int kTileCopiesMin = (KS8 && FMT == 0) ? 1 : 2;
    constexpr int kWaitTile1 = kTileCopiesMin | (7 << 4) | (15 << 8); // s_waitcnt vmcnt(min)
    static_assert(FMT != 0 || (RAW16 > NTHR && RAW16 - NTHR <= 64), "slot layout");
    static_assert(FMT == 0 || RAW16 == 2 * NTHR, "slot layout");
    __shared__ Smem<FMT> sm;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6); // uniform: keep it scalar
    const int qcol = lane & 31, g = lane >> 5;
    // SPLIT, KEY SPLIT: this wavefront's key subtile
    const int kh = SPLIT ? (wave >> 1) : KS8 ? (wave >> 2) : 0;

    // ---- workgroup -> (sequence, head, query tile).  Workgroups are dispatched round-robin over
    // the 8 XCDs; each XCD gets a contiguous set of heads (their K/V stay in its L2) and within
    // it the query tiles that see the most keys come first.
    const int n_qt = (a.M + QTF - 1) / QTF;
    const int BH = a.B * a.H;
    const int wg = blockIdx.x;
    int r, head_i;
    if (BH % 8 == 0) {
        const int hpx = BH / 8, slot = wg / 8;
        r = slot / hpx;
        head_i = (wg % 8) * hpx + slot % hpx;
    } else {
        r = wg / BH;
        head_i = wg % BH;
    }
    const int qt = n_qt - 1 - r;
    const int b = head_i / a.H, h = head_i % a.H;
    const int64_t head = head_i;

    auto kv_end_for = [&](int qrow) -> int { // keys [0, end) of the chunk visible to query qrow
        if (!a.causal)
            return a.n_kv;
        const int64_t e = a.q_pos0 + qrow - a.kv_pos0 + 1;
        return (int)(e < 0 ? 0 : (e > a.n_kv ? a.n_kv : e));
    };
    const int q_wg0 = qt * QTF;
    const int kv_end_wg = kv_end_for(min(q_wg0 + QTF, a.M) - 1);
    if (kv_end_wg <= 0)
        return; // the whole workgroup sees nothing of this chunk
    const int n_tiles = (kv_end_wg + KT - 1) / KT;

    // ---- this wavefront's 32-row query blocks: w and 7 - w of the tile (balances the causal
    // diagonal across wavefronts); SPLIT: block w & 1; NARROW: block w; KEY SPLIT: as w & 3
    int kv_end_b[NJ], kv_full_b[NJ], qi[NJ], lim[NJ];
    bool q_ok[NJ];
    int64_t row[NJ];
    // first query row of this wavefront's j-th block (wavefront-uniform)
    auto block_q0 = [&](int j) {
        return q_wg0 +
               WQ * (SPLIT ? (wave & 1) : NARROW ? wave : (j == 0 ? (wave & 3) : 7 - (wave & 3)));
    };
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int q0 = block_q0(j);
        const bool live = q0 < a.M;
        kv_end_b[j] = live ? kv_end_for(min(q0 + WQ, a.M) - 1) : 0;
        kv_full_b[j] = (q0 + WQ <= a.M) ? kv_end_for(q0) : 0;
        qi[j] = q0 + qcol;
        q_ok[j] = qi[j] < a.M;
        // last chunk key this lane's query sees (-1: none)
        lim[j] = q_ok[j] ? kv_end_for(qi[j]) - 1 : -1;
        row[j] = head * a.M + qi[j];
    }
    int kv_end_w = kv_end_b[0], kv_full_w = kv_full_b[0]; // kv_full_w: keys all rows see
#pragma unroll
    for (int j = 1; j < NJ; ++j) {
        kv_end_w = max(kv_end_w, kv_end_b[j]);
        kv_full_w = min(kv_full_w, kv_full_b[j]);
    }

    // ---- K/V tile pipeline: raw rows of tile t+2 are copied into LDS while tile t is computed
    // and tile t+1 is unpacked; one barrier per tile.
    const uint8_t *kbase = a.k + b * a.kv_seq_stride + h * a.kv_head_stride;
    const uint8_t *vbase = a.v + b * a.kv_seq_stride + h * a.kv_head_stride;
    // The range is rounded up to 16 bytes: the last 16-byte piece may hold up to 12 bytes past
    // the chunk, never past the 16-byte-aligned block that ends it (so never into another page);
    // those bytes belong to keys beyond n_kv, which are masked and get a zero V scale.
    const uint32_t head_bytes = ((uint32_t)a.n_kv * ROW + 15u) & ~15u;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase, head_bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase, head_bytes);
    // Raw rows are copied HBM -> LDS by buffer loads that write LDS directly (no registers, no
    // LDS store instructions): one instruction moves 16 bytes per lane to base + 16 * lane, so
    // each slot below covers 64 consecutive 16-byte pieces of one tensor per wavefront (the
    // buffer resource and the LDS base must be wavefront-uniform).
    //   Q8_0 (272 pieces per tensor): slot 0 = K piece tid, slot 1 = V piece tid, slot 2 = the
    //   16 remaining K pieces on wavefront 0 and the 16 remaining V pieces on wavefront 1.
    //   FP16 (512 pieces per tensor): slots 0, 1 = K pieces tid, tid + 256; slots 2, 3 = V.
    //   KEY SPLIT (512 threads): Q8_0 slot 0 = K piece tid on wavefronts 0-3 and V piece
    //   tid - 256 on 4-7, slot 1 = the 16 remaining K (wavefront 0) and V (wavefront 1) pieces;
    //   FP16 slot 0 = K piece tid, slot 1 = V piece tid.
    auto slot = [&](int sl, int &tensor, int &piece) -> bool {
        if constexpr (KS8 && FMT == 0) {
            if (sl == 0) {
                tensor = wave >> 2;
                piece = tid & (NTHR - 1);
                return true;
            }
            tensor = wave;
            piece = NTHR + lane;
            return wave < 2 && lane < RAW16 - NTHR;
        } else if constexpr (KS8) {
            tensor = sl;
            piece = tid;
            return true;
        } else if constexpr (FMT == 0) {
            if (sl < 2) {
                tensor = sl;
                piece = tid;
                return true;
            }
            tensor = wave;
            piece = NTHR + lane;
            return wave < 2 && lane < RAW16 - NTHR;
        } else {
            tensor = sl >> 1;
            piece = tid + NTHR * (sl & 1);
            return true;
        }
    };
    // raw rows of tile t into raw buffer buf; complete once vmcnt reaches 0
    auto fetch = [&](int t, int buf) {
#pragma unroll
        for (int sl = 0; sl < NPRE; ++sl) {
            int tensor, piece;
            if (slot(sl, tensor, piece)) {
                const uint32_t off = (uint32_t)t * (KT * ROW) + 16u * piece;
                uint8_t *dst = &sm.raw[buf][tensor][16 * (piece - lane)];
                const uint32_t base = __builtin_amdgcn_readfirstlane(
                    (uint32_t)(uintptr_t)(lds_void *)dst);
                dma16(tensor ? rv : rk, off, base);
            }
        }
    };
    // raw rows of buffer buf -> operand tile buf; keys from `valid` on lie past the chunk.
    // KEY SPLIT: K by wavefronts 0-3, V by 4-7 (each part over 256 threads).
    auto unpack = [&](int buf, int valid) {
        if constexpr (KS8) {
            if (wave < 4)
                unpack_tile<FMT, !CLEAN, 1>(sm.raw[buf][0], sm.raw[buf][1], sm.tile[buf], tid,
                                            valid);
            else
                unpack_tile<FMT, !CLEAN, 2>(sm.raw[buf][0], sm.raw[buf][1], sm.tile[buf],
                                            tid - NTHR, valid);
        } else {
            unpack_tile<FMT, !CLEAN>(sm.raw[buf][0], sm.raw[buf][1], sm.tile[buf], tid, valid);
        }
    };

    // Loads past the chunk read as zero, and operand tiles unpacked from raw rows past the last
    // tile are never read, so unpack runs unconditionally (no branches inside the tile loop's
    // scheduling regions); copies are skipped past the last tile.
    // Prologue: tile 0's copies, every row's Q and m, then tile 1's copies, all in flight
    // together; the resumed rows' l and O are loaded after it, their latency covered by the
    // first tile's QK work (they are first used by its rescale or PV products).
    fetch(0, 0);

    half8 qreg[NJ][4];
    floatx16 o[NJ][2];
    float l_part[NJ], m_top[NJ], m_ref[NJ], m_old[NJ];
    bool saw[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            o[j][0][v] = 0.f;
            o[j][1][v] = 0.f;
        }
        l_part[j] = 0.f;
        m_top[j] = -INFINITY; // running maximum of the logits, log2 units
        m_ref[j] = -INFINITY; // reference maximum of the exponentials, log2 units
        saw[j] = false;
        m_old[j] = -INFINITY;
        if (kv_end_b[j] > 0 && q_ok[j]) {
            const half8 *qrow = reinterpret_cast<const half8 *>(
                reinterpret_cast<const _Float16 *>(a.q) + row[j] * kHeadDim);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                qreg[j][kk] = qrow[2 * kk + g];
            // SPLIT, KEY SPLIT: only the first key subtile's wavefront resumes from the state;
            // the other starts empty and is merged in at the end
            if ((!KSPLIT || kh == 0) && !a.fresh)
                m_old[j] = a.m[row[j]];
        } else {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                qreg[j][kk] = half8{};
        }
    }
    // Tile 1's copies go last: at least kTileCopiesMin per thread, so waiting until at most
    // that many vector-memory loads are outstanding (they complete in order) leaves only those
    // in flight while tile 0 is unpacked; they have landed before the barrier after it.
    if (n_tiles > 1) {
        fetch(1, 1);
        __builtin_amdgcn_s_waitcnt(kWaitTile1);
    } else {
        __builtin_amdgcn_s_waitcnt(0);
    }
    __syncthreads();
    unpack(0, a.n_kv);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NJ; ++j)
        if (m_old[j] != -INFINITY) {
            m_top[j] = m_old[j] * kLog2e;
            m_ref[j] = m_top[j];
        }
    // l and O of the resumed rows, this head's rows of the state as buffers: lanes of rows
    // that are empty (or whose l another lane reads) address past the range and read 0,
    // so the loads need no branch
    const __amdgpu_buffer_rsrc_t rs_o = make_rsrc(a.o + head * a.M * kHeadDim,
                                                  (uint32_t)a.M * kHeadDim * 4u);
    const __amdgpu_buffer_rsrc_t rs_l = make_rsrc(a.l + head * a.M, (uint32_t)a.M * 4u);
    const __amdgpu_buffer_rsrc_t rs_m = make_rsrc(a.m + head * a.M, (uint32_t)a.M * 4u);
    // past-the-end offset: beyond the largest range (n_q < 2^24 rows of 256 bytes, checked on
    // the host) even with the 240 bytes a row's last piece adds, and without wrapping
    constexpr uint32_t kNoRow = 0xFFFFFF00u;
    auto load_resumed = [&]() {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const bool res = m_old[j] != -INFINITY;
            const uint32_t ob = res ? (uint32_t)qi[j] * (kHeadDim * 4u) : kNoRow;
            const uint32_t lb = (res && g == 0) ? (uint32_t)qi[j] * 4u : kNoRow;
            l_part[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs_l, lb, 0, 0));
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const u32x4 x = load16(rs_o, ob + 16u * (2 * k + g));
                const u32x4 y = load16(rs_o, ob + 16u * (8 + 2 * k + g));
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    o[j][0][4 * k + e] = __uint_as_float(x[e]);
                    o[j][1][4 * k + e] = __uint_as_float(y[e]);
                }
            }
        }
    };

    auto tile = [&](const int t, auto jlo_c) {
        // raw buffer t&1 was unpacked in the previous interval; no copies past the last tile
        // (for a workgroup on the causal diagonal they would be real reads)
        if (t + 2 < n_tiles)
            fetch(t + 2, t & 1);
        const KvTile<FMT> &T = sm.tile[t & 1];
        const int key0 = t * KT;
        // tile t+1 is unpacked from its raw rows in every branch: the same barrier interval
        // that reads operand buffer t&1 writes buffer (t+1)&1
        // the tile's work for blocks JLO .. NJ-1 (JLO = 1: block 0 sees no key of this tile)
        auto compute = [&](auto jlo_c) {
            constexpr int JLO = decltype(jlo_c)::value;
                // S^T = K Q^T: lane (qcol, g) holds
                // S^T[key 32*sub + 8*(v/4) + 4*g + v%4][query qcol] in s[j][si][v], sub the
                // si-th key subtile this wavefront covers.  Q8_0: the first block's products (dims
                // 0-31) are scaled by kr before the second block's are added.
                floatx16 s[NJ][NS];
#pragma unroll
                for (int j = JLO; j < NJ; ++j)
#pragma unroll
                    for (int si = 0; si < NS; ++si)
#pragma unroll
                        for (int v = 0; v < 16; ++v)
                            s[j][si][v] = 0.f;
#pragma unroll
                for (int half = 0; half < 2; ++half)
#pragma unroll
                    for (int si = 0; si < NS; ++si) {
                        const int sub = KSPLIT ? kh : si;
                        const int krow = (32 * sub + qcol) * KP + 8 * g;
                        if (FMT == 0 && half == 1) {
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const float4 r4 = *reinterpret_cast<const float4 *>(
                                    &T.kr[32 * sub + 8 * i + 4 * g]);
#pragma unroll
                                for (int j = JLO; j < NJ; ++j) {
                                    s[j][si][4 * i + 0] *= r4.x;
                                    s[j][si][4 * i + 1] *= r4.y;
                                    s[j][si][4 * i + 2] *= r4.z;
                                    s[j][si][4 * i + 3] *= r4.w;
                                }
                            }
                        }
#pragma unroll
                        for (int kk = 2 * half; kk < 2 * half + 2; ++kk) {
                            const half8 ak = *reinterpret_cast<const half8 *>(&T.k[krow + 16 * kk]);
#pragma unroll
                            for (int j = JLO; j < NJ; ++j)
                                s[j][si] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ak, qreg[j][kk],
                                                                                 s[j][si], 0, 0, 0);
                        }
                    }
                // independent VALU work for the matrix instructions above to overlap with
                unpack((t + 1) & 1, a.n_kv - (t + 1) * KT);

                // u = S*log2(e)/8 - ref, the exponent relative to the reference maximum before
                // this tile (0 while it is -inf)
                float base[NJ];
#pragma unroll
                for (int j = JLO; j < NJ; ++j)
                    base[j] = (m_ref[j] == -INFINITY) ? 0.f : m_ref[j];
#pragma unroll
                for (int si = 0; si < NS; ++si) {
                    const int sub = KSPLIT ? kh : si;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float4 m4 = {kScaleLog2, kScaleLog2, kScaleLog2, kScaleLog2};
                        if constexpr (FMT == 0)
                            m4 = *reinterpret_cast<const float4 *>(&T.km[32 * sub + 8 * i + 4 * g]);
#pragma unroll
                        for (int j = JLO; j < NJ; ++j) {
                            const int e = 4 * i;
                            s[j][si][e + 0] = __builtin_fmaf(s[j][si][e + 0], m4.x, -base[j]);
                            s[j][si][e + 1] = __builtin_fmaf(s[j][si][e + 1], m4.y, -base[j]);
                            s[j][si][e + 2] = __builtin_fmaf(s[j][si][e + 2], m4.z, -base[j]);
                            s[j][si][e + 3] = __builtin_fmaf(s[j][si][e + 3], m4.w, -base[j]);
                        }
                    }
                }

                // The 32-key subtiles that some row of a block cannot wholly see (causal diagonal,
                // ragged chunk end, padding rows) are masked element by element; the common case
                // skips this with one wavefront-uniform test.
                if (key0 + KT > kv_full_w) {
#pragma unroll
                    for (int j = JLO; j < NJ; ++j) {
                        // key key0 + 32*sub + 8*(v/4) + 4*g + v%4 is visible iff it is <= lim
                        const int rel = lim[j] - key0 - 4 * g;
#pragma unroll
                        for (int si = 0; si < NS; ++si) {
                            const int sub = KSPLIT ? kh : si;
                            if (key0 + 32 * sub + 32 > kv_full_b[j]) {
#pragma unroll
                                for (int v = 0; v < 16; ++v)
                                    s[j][si][v] = (32 * sub + 8 * (v >> 2) + (v & 3) <= rel)
                                                      ? s[j][si][v] : -INFINITY;
                            }
                        }
                    }
                }
                bool need_any = false;
                float mx[NJ];
                bool need[NJ];
#pragma unroll
                for (int j = JLO; j < NJ; ++j) {
                    if constexpr (NS == 2) {
                        float ma = vmax3(s[j][0][0], s[j][0][1], s[j][0][2]);
                        float mb = vmax3(s[j][1][0], s[j][1][1], s[j][1][2]);
#pragma unroll
                        for (int v = 3; v < 15; v += 2) {
                            ma = vmax3(ma, s[j][0][v], s[j][0][v + 1]);
                            mb = vmax3(mb, s[j][1][v], s[j][1][v + 1]);
                        }
                        mx[j] = vmax3(ma, mb, fmaxf(s[j][0][15], s[j][1][15]));
                    } else {
                        float ma = vmax3(s[j][0][0], s[j][0][1], s[j][0][2]);
#pragma unroll
                        for (int v = 3; v < 15; v += 2)
                            ma = vmax3(ma, s[j][0][v], s[j][0][v + 1]);
                        mx[j] = fmaxf(ma, s[j][0][15]);
                    }
                    mx[j] = half_swap_max(mx[j]); // tile maximum of u for this query row
                    m_top[j] = fmaxf(m_top[j], base[j] + mx[j]);
                    saw[j] = saw[j] || (mx[j] != -INFINITY);
                    // raise the reference when the tile's maximum exceeds it by more than kTau (or
                    // when it is still -inf and the row saw a key)
                    need[j] = mx[j] > (m_ref[j] == -INFINITY ? -INFINITY : kTau);
                    need_any = need_any || need[j];
                }
                if (__builtin_amdgcn_ballot_w64(need_any)) {
#pragma unroll
                    for (int j = JLO; j < NJ; ++j) {
                        const float delta = need[j] ? mx[j] : 0.f; // new ref = base + delta
                        // rows whose reference is still -inf hold l = 0 and O = 0: only rows
                        // with a finite reference that moves need their sums rescaled (the first
                        // tile of a fresh state has none)
                        if (__builtin_amdgcn_ballot_w64(need[j] && m_ref[j] != -INFINITY)) {
                            const float alpha = (m_ref[j] == -INFINITY)
                                                    ? 0.f : __builtin_amdgcn_exp2f(-delta);
                            l_part[j] *= alpha;
                            o[j][0] *= alpha;
                            o[j][1] *= alpha;
                        }
                        if (need[j])
                            m_ref[j] = base[j] + delta;
#pragma unroll
                        for (int si = 0; si < NS; ++si)
                            s[j][si] -= delta;
                    }
                }
                // per query block: P = exp2(u) (l sums the FP32 values), P to FP16, then
                // O^T += V^T P^T.  Block 0's products overlap block 1's exponentials.
#pragma unroll
                for (int j = JLO; j < NJ; ++j) {
                    float ls[4]; // four partial sums: shorter chains
                    half8 p16[NS][2];
#pragma unroll
                    for (int si = 0; si < NS; ++si) {
#pragma unroll
                        for (int v = 0; v < 16; ++v) {
                            const float p = __builtin_amdgcn_exp2f(s[j][si][v]);
                            s[j][si][v] = p;
                            // the first four start the sums (not 0 + p: the compiler may not
                            // drop that addition, which would turn -0 into +0)
                            ls[v & 3] = (si == 0 && v < 4) ? p : ls[v & 3] + p;
                        }
                        p16[si][0] = to_half8(s[j][si], 0);
                        p16[si][1] = to_half8(s[j][si], 8);
                    }
                    l_part[j] += (ls[0] + ls[1]) + (ls[2] + ls[3]);
                    // the V tile's key order matches the accumulator layout
#pragma unroll
                    for (int si = 0; si < NS; ++si)
#pragma unroll
                        for (int tt = 0; tt < 2; ++tt) {
                            const int sub = KSPLIT ? kh : si;
                            const int pos = 32 * sub + 16 * tt + 8 * g;
                            const half8 a0 =
                                *reinterpret_cast<const half8 *>(&T.vt[qcol * VP + pos]);
                            const half8 a1 =
                                *reinterpret_cast<const half8 *>(&T.vt[(32 + qcol) * VP + pos]);
                            o[j][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, p16[si][tt],
                                                                             o[j][0], 0, 0, 0);
                            o[j][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, p16[si][tt],
                                                                             o[j][1], 0, 0, 0);
                        }
                }
        };
        if (key0 < kv_end_w) {
            compute(jlo_c);
        } else {
            unpack((t + 1) & 1, a.n_kv - (t + 1) * KT);
        }
        __builtin_amdgcn_s_waitcnt(0); // raw rows of tile t+2 have landed before the barrier
        __syncthreads();
    };
    // The first tile is peeled: the state loads are issued right before its copies, so the
    // wait in front of their first use leaves those copies in flight.
    load_resumed();
    tile(0, std::integral_constant<int, 0>{});
    if constexpr (NJ == 2 && (CLEAN || FMT == 1)) {
        // On the causal diagonal a wavefront's first block (the lower rows) stops seeing keys
        // before its second block does; from then on the tiles run for the second block only
        // (the work left out would be all masked).  Each wavefront runs every tile interval, so
        // the barriers still match.  (Not in the masked Q8_0 unpack form: there the second loop
        // would push the kernel past 256 VGPRs.)
        int t_two = n_tiles;
        if (kv_end_b[1] > kv_end_b[0])
            t_two = max(1, (kv_end_b[0] + KT - 1) / KT);
        int t = 1;
        for (; t < t_two; ++t)
            tile(t, std::integral_constant<int, 0>{});
        for (; t < n_tiles; ++t)
            tile(t, std::integral_constant<int, 1>{});
    } else {
        for (int t = 1; t < n_tiles; ++t)
            tile(t, std::integral_constant<int, 0>{});
    }

    // The key-splitting forms merge the two key subtiles' states of each block: the second
    // subtile's wavefront (kh = 1) leaves its per-lane state in LDS (the loop's last barrier has
    // retired every use of the tile buffers), the first (kh = 0, same lanes, same block) folds it
    // in.
    auto stash = [&](int j, float *xb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            xb[v] = o[j][0][v];
            xb[16 + v] = o[j][1][v];
        }
        xb[32] = l_part[j];
        xb[33] = m_ref[j];
        xb[34] = m_top[j];
        xb[35] = saw[j] ? 1.f : 0.f;
    };
    auto fold = [&](int j, const float *xb) {
        const float mb = xb[33];
        if (mb != -INFINITY) { // the other subtile's state is not empty
            const float ma = m_ref[j];
            const float mn = fmaxf(ma, mb);
            const float fa = (ma == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ma - mn);
            const float fb = __builtin_amdgcn_exp2f(mb - mn);
            // one product, then one fused multiply-add, written out so that every instantiation
            // rounds the merge of the two key halves the same way
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                o[j][0][v] = __builtin_fmaf(xb[v], fb, o[j][0][v] * fa);
                o[j][1][v] = __builtin_fmaf(xb[16 + v], fb, o[j][1][v] * fa);
            }
            l_part[j] = __builtin_fmaf(xb[32], fb, l_part[j] * fa);
            m_ref[j] = mn;
        }
        m_top[j] = fmaxf(m_top[j], xb[34]);
        saw[j] = saw[j] || xb[35] != 0.f;
    };
    if constexpr (SPLIT) {
        static_assert(sizeof(Smem<FMT>) >= 2 * 64 * 36 * sizeof(float), "merge area");
        float *xb = reinterpret_cast<float *>(&sm) + ((wave & 1) * 64 + lane) * 36;
        if (kh == 1)
            stash(0, xb);
        __syncthreads();
        if (kh == 0)
            fold(0, xb);
    }
    if constexpr (KS8) {
        // one block at a time; the barrier after each pass retires its reads before the area is
        // reused (by the next pass, then by the write-back's staging)
        static_assert(sizeof(Smem<FMT>) >= 4 * 64 * 36 * sizeof(float), "merge area");
        float *xb = reinterpret_cast<float *>(&sm) + ((wave & 3) * 64 + lane) * 36;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            if (kh == 1)
                stash(j, xb);
            __syncthreads();
            if (kh == 0)
                fold(j, xb);
            __syncthreads();
        }
    }

    // ---- write back the rows that saw at least one key, renormalised to the true maximum.
    // Each wavefront stages its 32-row block in LDS (its own region, past the area the merge
    // above uses) and stores whole rows: 4 contiguous rows (1 KiB) per store instruction, instead
    // of 32-byte pieces of 32 rows.  A row's write flag travels with it.
    // With a.out set, the rows whose query position lies inside the chunk are final (in a
    // causal pass over chunks in ascending key order no later key is visible to them): their
    // out and lse are written as the finalize kernel would from the state just stored (the same
    // FP32 values, the same reciprocal, product and logarithm), flag 2 instead of 1.
    constexpr int kStagePitch = 68;                                // floats per staged row
    constexpr int kStageFloats = WQ * kStagePitch + 3 * WQ;        // rows, 2 offsets, final 1/l
    constexpr int kStageBase = 2 * 64 * 36;                        // floats
    static_assert(sizeof(Smem<FMT>) >= 4 * (kStageBase + 4 * kStageFloats), "staging area");
    float *stg = reinterpret_cast<float *>(&sm) + kStageBase + wave * kStageFloats;
    // per staged row: its byte offset in the state's O and in out (past the range where the row
    // is not written), and a final row's 1/l
    uint32_t *stg_off = reinterpret_cast<uint32_t *>(stg + WQ * kStagePitch);
    uint32_t *stg_oo = stg_off + WQ;
    float *stg_l = reinterpret_cast<float *>(stg_oo + WQ);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        if (kv_end_b[j] > 0 && (!KSPLIT || kh == 0)) { // uniform per wavefront
            const float l_tot = half_swap_sum(l_part[j]);
            const bool wr = q_ok[j] && saw[j];
            const float rr = wr ? __builtin_amdgcn_exp2f(m_ref[j] - m_top[j]) : 0.f;
            const int64_t pos = a.q_pos0 + qi[j]; // this lane's query position
            const bool fin = a.out && wr && pos >= a.kv_pos0 && pos < a.kv_pos0 + a.n_kv;
            // m and l are stored for the rows that saw a key (a fresh state: for every row,
            // m = -inf and l = 0 where none was seen), except final rows whose state is dead
            const bool st_ml = q_ok[j] && (saw[j] || a.fresh) && !(fin && a.final_out_only);
            // does the block hold a final row (wavefront-uniform)?
            const int64_t p0 = a.q_pos0 + block_q0(j);
            const bool fin_block = a.out && p0 + WQ > a.kv_pos0 && p0 < a.kv_pos0 + a.n_kv;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                *reinterpret_cast<float4 *>(&stg[qcol * kStagePitch + 8 * k + 4 * g]) =
                    make_float4(o[j][0][4 * k] * rr, o[j][0][4 * k + 1] * rr,
                                o[j][0][4 * k + 2] * rr, o[j][0][4 * k + 3] * rr);
                *reinterpret_cast<float4 *>(&stg[qcol * kStagePitch + 32 + 8 * k + 4 * g]) =
                    make_float4(o[j][1][4 * k] * rr, o[j][1][4 * k + 1] * rr,
                                o[j][1][4 * k + 2] * rr, o[j][1][4 * k + 3] * rr);
            }
            // rows that are not written address past the head's range, where buffer stores
            // are dropped
            const uint32_t q0 = (uint32_t)block_q0(j);
            const float m_st = m_top[j] * kLn2, l_st = l_tot * rr; // the stored m and l
            // the lane that owns a row stages where its state row and its output row go: the
            // state of a row that saw a key unless it is final and its state dead, the output of
            // a final row
            if (g == 0) {
                const uint32_t rq = q0 + (uint32_t)qcol;
                stg_off[qcol] = (wr && !(fin && a.final_out_only)) ? rq * (kHeadDim * 4u) : kNoRow;
                stg_oo[qcol] = (wr && fin) ? rq * (kHeadDim * 2u) : kNoRow;
                // the final rows' reciprocal of l, formed once by the lane that owns the row
                if (fin_block)
                    stg_l[qcol] = final_inv_l(l_st);
            }
            const uint32_t ml_off = (st_ml && g == 0) ? (q0 + qcol) * 4u : kNoRow;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m_st), rs_m, ml_off, 0,
                                                  kStoreThrough);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(l_st), rs_l, ml_off, 0,
                                                  kStoreThrough);
            if (fin_block && a.lse)
                __builtin_amdgcn_raw_buffer_store_b32(
                    __float_as_uint(m_st + logf(l_st)),
                    make_rsrc(a.lse + head * a.M, (uint32_t)a.M * 4u),
                    (fin && g == 0) ? (q0 + qcol) * 4u : kNoRow, 0, kStoreThrough);
            // the same wavefront reads back what it wrote (LDS keeps a wavefront's order): all
            // rows and offsets first, so the LDS reads overlap, then the stores
            u32x4 vv[WQ / 4];
            uint32_t off[WQ / 4];
#pragma unroll
            for (int i = 0; i < WQ / 4; ++i) {
                const int r = 4 * i + (lane >> 4), c = lane & 15;
                vv[i] = *reinterpret_cast<const u32x4 *>(&stg[r * kStagePitch + 4 * c]);
                off[i] = stg_off[r] + 16u * c; // past the range stays past it: kNoRow + 240
            }
#pragma unroll
            for (int i = 0; i < WQ / 4; ++i)
                __builtin_amdgcn_raw_buffer_store_b128(vv[i], rs_o, off[i], 0, kStoreThrough);
            if (fin_block) {
                // out = O / l as final_out forms it, 4 values per lane and row
                const __amdgpu_buffer_rsrc_t rs_out =
                    make_rsrc(reinterpret_cast<_Float16 *>(a.out) + head * a.M * kHeadDim,
                              (uint32_t)a.M * (kHeadDim * 2u));
#pragma unroll
                for (int i = 0; i < WQ / 4; ++i) {
                    const int r = 4 * i + (lane >> 4), c = lane & 15;
                    const float rl = stg_l[r];
                    const uint32_t oo = stg_oo[r] + 8u * c;
                    const half4 h = {final_out(__uint_as_float(vv[i][0]), rl),
                                     final_out(__uint_as_float(vv[i][1]), rl),
                                     final_out(__uint_as_float(vv[i][2]), rl),
                                     final_out(__uint_as_float(vv[i][3]), rl)};
                    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, h), rs_out,
                                                          oo, 0, kStoreThrough);
                }
            }
        }
    }
}

// m = -inf, l = 0: four rows per thread, as one 16-byte store per array when both arrays are
// 16-byte aligned (the usual case), else four 4-byte stores
__global__ __launch_bounds__(256) void state_init_kernel(float *m, float *l, int64_t n_rows)
{
    const int64_t i = 4 * ((int64_t)blockIdx.x * 256 + threadIdx.x);
    if (i >= n_rows)
        return;
    const bool vec = ((reinterpret_cast<uintptr_t>(m) | reinterpret_cast<uintptr_t>(l)) & 15) == 0;
    if (vec && i + 4 <= n_rows) {
        *reinterpret_cast<float4 *>(m + i) = make_float4(-INFINITY, -INFINITY, -INFINITY,
                                                         -INFINITY);
        *reinterpret_cast<float4 *>(l + i) = make_float4(0.f, 0.f, 0.f, 0.f);
        return;
    }
    for (int64_t r = i; r < i + 4 && r < n_rows; ++r) {
        m[r] = -INFINITY;
        l[r] = 0.f;
    }
}

// out = O / l (final_inv_l, final_out); lse = m + ln l.  Eight lanes per row, 8 values each.
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
        const float rl = final_inv_l(lv);
        const float4 x = o[row * 16 + 2 * part];
        const float4 y = o[row * 16 + 2 * part + 1];
        res[0] = final_out(x.x, rl); res[1] = final_out(x.y, rl);
        res[2] = final_out(x.z, rl); res[3] = final_out(x.w, rl);
        res[4] = final_out(y.x, rl); res[5] = final_out(y.y, rl);
        res[6] = final_out(y.z, rl); res[7] = final_out(y.w, rl);
        if (part == 0 && lse)
            lse[row] = mv + logf(lv);
    }
    out[row * 8 + part] = res;
}

// Merge partial state b into partial state a, row by row: m' = max(m_a, m_b), then l and O of
// each side are rescaled by e^(m - m') and added (the chunk rescale of "Out-of-Core Flash
// Streaming & Speculative Decode (1M Context)", Sec. 3, with b's summary in the chunk's place).
// An empty b (m = -inf) leaves a untouched; an empty a takes b.  Eight lanes per row, eight O
// values each; all lanes of a row read its m and l before lane 0 writes them.
__global__ __launch_bounds__(256) void merge_kernel(float *__restrict__ ma, float *__restrict__ la,
                                                    float4 *__restrict__ oa,
                                                    const float *__restrict__ mb,
                                                    const float *__restrict__ lb,
                                                    const float4 *__restrict__ ob,
                                                    int64_t n_rows)
{
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = gid >> 3;
    const int part = (int)(gid & 7);
    if (row >= n_rows)
        return;
    const float m2 = mb[row];
    if (m2 == -INFINITY)
        return;
    const float m1 = ma[row];
    const float4 y0 = ob[row * 16 + 2 * part], y1 = ob[row * 16 + 2 * part + 1];
    float4 r0, r1;
    float mn, ln;
    if (m1 == -INFINITY) {
        r0 = y0;
        r1 = y1;
        mn = m2;
        ln = lb[row];
    } else {
        mn = fmaxf(m1, m2);
        const float fa = expf(m1 - mn), fb = expf(m2 - mn);
        const float4 x0 = oa[row * 16 + 2 * part], x1 = oa[row * 16 + 2 * part + 1];
        r0 = make_float4(x0.x * fa + y0.x * fb, x0.y * fa + y0.y * fb, x0.z * fa + y0.z * fb,
                         x0.w * fa + y0.w * fb);
        r1 = make_float4(x1.x * fa + y1.x * fb, x1.y * fa + y1.y * fb, x1.z * fa + y1.z * fb,
                         x1.w * fa + y1.w * fb);
        ln = la[row] * fa + lb[row] * fb;
    }
    oa[row * 16 + 2 * part] = r0;
    oa[row * 16 + 2 * part + 1] = r1;
    if (part == 0) {
        ma[row] = mn;
        la[row] = ln;
    }
}

} // namespace

hipError_t launch_state_init(float *m, float *l, int64_t n_rows, hipStream_t s)
{
    const int64_t grid = (n_rows + 1023) / 1024;
    hipLaunchKernelGGL(state_init_kernel, dim3((unsigned)grid), dim3(256), 0, s, m, l, n_rows);
    return hipGetLastError();
}

// Workgroup slots of the current device: 2 per compute unit (the kernel holds 2 workgroups of
// 4 wavefronts per CU); 0 when it cannot be read.
static int workgroup_slots()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 0;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        v = 2 * cus;
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

// Launches the query tiles whose rows see some key of the chunk: with the causal mask, rows before
// position kv_pos0 see none, and the kernel maps the first workgroups to the last query tiles, so
// the grid ends at the first tile that holds a row at or past kv_pos0.
template <int FMT, bool CLEAN>
static void launch_form(const AccumulateArgs &a, int form, hipStream_t s)
{
    const int rows = form == kSplit ? 2 * WQ : form == kNarrow ? QT / 2 : QT;
    const int64_t n_qt = (a.M + rows - 1) / rows;
    int64_t first_row = 0;
    if (a.causal && a.kv_pos0 > a.q_pos0)
        first_row = a.kv_pos0 - a.q_pos0;
    if (first_row >= a.M)
        return; // no row sees the chunk
    const dim3 grid((unsigned)((n_qt - first_row / rows) * a.B * a.H));
    switch (form) {
    case kSplit:
        hipLaunchKernelGGL((accumulate_kernel<FMT, kSplit, CLEAN>), grid, dim3(NTHR), 0, s, a);
        break;
    case kNarrow:
        hipLaunchKernelGGL((accumulate_kernel<FMT, kNarrow, CLEAN>), grid, dim3(NTHR), 0, s, a);
        break;
    case kKeySplit:
        hipLaunchKernelGGL((accumulate_kernel<FMT, kKeySplit, CLEAN>), grid, dim3(2 * NTHR), 0, s,
                           a);
        break;
    default:
        hipLaunchKernelGGL((accumulate_kernel<FMT, kWide, CLEAN>), grid, dim3(NTHR), 0, s, a);
    }
}

hipError_t launch_accumulate(const AccumulateArgs &a, int kv_dtype, hipStream_t s)
{
    // The tile form.  Up to 64 query rows (two blocks): split the keys of every tile between
    // wavefront pairs.  Otherwise 256-row workgroups, unless the launch would not fill the chip's
    // workgroup slots (2 per compute unit):
    //   * where the causal diagonal crosses the chunk so that the first row sees less than half
    //     of what the last row sees, the query tiles' work is uneven and the launch lasts as
    //     long as the tile that sees the most; 128-row workgroups halve that tile's work per key,
    //     and where even 64-row workgroups would fill at most half the slots (the last chunk of
    //     a short causal prefill, which only the diagonal rows see), those with key-split
    //     wavefront pairs quarter it;
    //   * otherwise the load is (nearly) even; with at most one workgroup per compute unit, the
    //     8-wavefront key-split form gives every SIMD two wavefronts while each K/V tile is
    //     still unpacked once for 256 rows.
    // Workgroup counts are those launched: the query tiles that hold a row seeing the chunk.
    // a.form, when set, fixes the form for more than 64 rows.
    const int slots = workgroup_slots();
    int64_t first_row = 0;
    if (a.causal && a.kv_pos0 > a.q_pos0)
        first_row = std::min<int64_t>(a.kv_pos0 - a.q_pos0, a.M);
    auto launched = [&](int rows) {
        return (int64_t)((a.M + rows - 1) / rows - first_row / rows) * a.B * a.H;
    };
    const int64_t wide = launched(QT);
    // keys of the chunk the first and the last query row see (at least one for the first)
    auto clamp_keys = [&](int64_t n, int64_t lo) {
        return std::min<int64_t>(std::max(n, lo), a.n_kv);
    };
    const int64_t seen_lo = clamp_keys(a.q_pos0 - a.kv_pos0 + 1, 1);
    const int64_t seen_hi = clamp_keys(a.q_pos0 + a.M - a.kv_pos0, 0);
    const bool uneven = a.causal && 2 * seen_lo < seen_hi;
    int form = kWide;
    if (a.M <= 2 * WQ)
        form = kSplit;
    else if (wide < slots) {
        if (uneven)
            form = 2 * launched(2 * WQ) <= slots ? kSplit : kNarrow;
        else
            form = 2 * wide <= slots ? kKeySplit : kWide;
    }
    if (a.M > 2 * WQ) {
        if (a.form == kFormNarrow)
            form = kNarrow;
        else if (a.form == kFormWide)
            form = kWide;
        else if (a.form == kFormKeySplit)
            form = kKeySplit;
        else if (a.form == kFormSplit)
            form = kSplit;
    }
    if (kv_dtype != 0)
        launch_form<1, true>(a, form, s); // FP16 rows: 128 bytes, always clean
    else if (a.n_kv % 4 == 0)
        launch_form<0, true>(a, form, s);
    else
        launch_form<0, false>(a, form, s);
    return hipGetLastError();
}

hipError_t launch_merge(float *ma, float *la, float *oa, const float *mb, const float *lb,
                        const float *ob, int64_t n_rows, hipStream_t s)
{
    const int64_t grid = (n_rows * 8 + 255) / 256;
    hipLaunchKernelGGL(merge_kernel, dim3((unsigned)grid), dim3(256), 0, s, ma, la,
                       reinterpret_cast<float4 *>(oa), mb, lb,
                       reinterpret_cast<const float4 *>(ob), n_rows);
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
