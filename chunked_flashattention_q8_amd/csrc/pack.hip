// Q8_0 pack kernel ("Core Architecture & The 4-Brick Pipeline", Sec. 5, block_q8_0: 32 int8
// values plus one FP16 scale, 34 bytes, 8-bit symmetric).
//
// HBM-bound: each 32-value block reads 128 bytes and writes 34.  Eight consecutive lanes own one
// block and each loads one 16-byte float4, so a wavefront reads 1 KiB of contiguous input per
// instruction; every lane handles two blocks, 256 float4 apart, with both loads in flight.  Loads
// and stores are non-temporal (the source is read once; the packed rows are streamed out).  The
// block's largest magnitude is reduced over the eight lanes (DPP), every lane derives the same FP16
// scale, quantises its four values and writes them with one 4-byte store (block starts are only
// 2-byte aligned: 34 * k).
//
// Arithmetic (bit-exact with the CPU oracle): d = amax / 127 correctly rounded in FP32
// (div127); d16 = FP16(d), round to nearest even; q = round(x / d16) with a correctly rounded
// FP32 division and halves away from zero, clamped to [-127, 127]; an all-zero block gives
// d16 = 0 and q = 0.  The quotients are formed from the product with the reciprocal of d16 and
// fall back to the division where that could round differently (see quantise4_fast, quantise).
#include <hip/hip_fp16.h>

#include "q8attn_internal.h"

namespace q8a {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32_a2 __attribute__((aligned(2)));

// Lane exchange within rows of 16 lanes (DPP).  Every lane of the wavefront is active where
// these are used, so every source lane is valid.
constexpr int kDppQuadSwap1 = 0xb1;  // quad_perm [1, 0, 3, 2]: lane i takes lane i ^ 1
constexpr int kDppQuadSwap2 = 0x4e;  // quad_perm [2, 3, 0, 1]: lane i takes lane i ^ 2
constexpr int kDppHalfMirror = 0x141; // row_half_mirror: lane i of each 8 takes lane 7 - i
template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// a / 127 correctly rounded (FP32, round to nearest even) for every finite a >= 0: the product
// with the rounded reciprocal, then one correction with the exact residual a - 127 q0 (an FMA).
// This form was checked against the IEEE division for all 2^31 - 2^23 non-negative finite FP32
// values, subnormals and zero included: no value differs.
__device__ __forceinline__ float div127(float a)
{
    constexpr float kInv127 = 1.0f / 127.0f; // 0x1.020408p-7
    const float q0 = a * kInv127;
    const float r = __builtin_fmaf(-q0, 127.0f, a);
    float d = __builtin_fmaf(r, kInv127, q0);
    // d is rounded to FP32 here: an empty asm keeps the compiler from merging the FMA with the
    // later conversion to FP16 into one instruction that would round only once
    asm("" : "+v"(d));
    return d;
}

// round(x / dh), halves away from zero, clamped to [-127, 127], with x / dh the correctly
// rounded FP32 quotient z'.  rdh is the hardware reciprocal of dh (relative error at most 2^-23):
// y = fl(x * rdh) differs from the exact quotient z by at most (2^-23 + 2^-24 + 2^-47) |z|, and z'
// from z by at most 2^-24 |z|.  With dh = FP16(amax / 127) (zero excepted) |z| < 256, so y and z'
// differ by less than 2^-14 and round to the same integer unless y lies within 2^-14 of a
// half-integer.  Such values (|frac(|y|) - 1/2| <= 2^-13: twice the bound, about 1 in 4000) and
// any |y| >= 255 take the correctly rounded division instead.  This is the general form, used for
// the blocks the fast form below leaves out.
__device__ __forceinline__ int quantise(float x, float dh, float rdh)
{
    if (dh == 0.0f)
        return 0;
    float y = x * rdh;
    float ay = fabsf(y);
    float ti = truncf(ay), fr = ay - ti; // exact for ay < 2^23
    if (fabsf(fr - 0.5f) <= 0x1p-13f || ay >= 255.0f) {
        y = __fdiv_rn(x, dh);
        ay = fabsf(y);
        ti = truncf(ay);
        fr = ay - ti;
    }
    const float q = fminf(ti + (fr >= 0.5f ? 1.0f : 0.0f), 127.0f);
    return (int)copysignf(q, y);
}

// The fast form for one lane's four values of a block whose scale dh is a normal FP16 number
// (dh >= 2^-14).  Then |x| <= amax <= 127 dh (1 + 2^-11) and every exact product x * rdh has
// magnitude below 127.1, so no clamp is needed.  f = fma(x, rdh, 1.5 * 2^23) rounds the exact
// product to the nearest integer r (ties to even) and holds r + 1.5 * 2^23 in the binade whose
// spacing is 1: the low byte of f's bits is r as a two's-complement byte.  d = fma(x, rdh, -r)
// is the product's distance from r (within 2^-25); where |d| >= 1/2 - 2^-13 the product lies
// within 2^-13 of a half-integer (the window of quantise above) and the lane reports it.
// Everywhere else the product, the exact quotient and the correctly rounded quotient are more
// than 2^-14 from a half-integer and round to the same r.  Returns the four bytes q0..q3 of the
// block's little-endian int8 sequence.
__device__ __forceinline__ uint32_t quantise4_fast(float4 v, float rdh, bool &near_tie)
{
    constexpr float kRound = 0x1.8p23f;
    const float f0 = __builtin_fmaf(v.x, rdh, kRound), f1 = __builtin_fmaf(v.y, rdh, kRound);
    const float f2 = __builtin_fmaf(v.z, rdh, kRound), f3 = __builtin_fmaf(v.w, rdh, kRound);
    const float d0 = __builtin_fmaf(v.x, rdh, kRound - f0);
    const float d1 = __builtin_fmaf(v.y, rdh, kRound - f1);
    const float d2 = __builtin_fmaf(v.z, rdh, kRound - f2);
    const float d3 = __builtin_fmaf(v.w, rdh, kRound - f3);
    const float dm = fmaxf(fmaxf(fabsf(d0), fabsf(d1)), fmaxf(fabsf(d2), fabsf(d3)));
    near_tie = dm >= 0.5f - 0x1p-13f;
    const uint32_t lo = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x04000c0cu);
    return lo | hi;
}

// Each lane packs its quarter of U blocks (U x 256 consecutive float4 per workgroup); the U loads
// are issued before any is used.  blockIdx.y selects a run of n_blocks blocks (one (sequence,
// head) pair of an appended chunk: its source at x + y * n_blocks * 8 float4, its destination
// at dst + (y / n_heads) * seq_stride + (y % n_heads) * head_stride) and blockIdx.z the tensor
// (K from x / dst, V from x2 / dst2); a flat pack is the single run y = z = 0.
template <int U>
__global__ __launch_bounds__(256) void q8_0_pack_kernel(const float4 *__restrict__ x,
                                                         uint8_t *__restrict__ dst,
                                                         int64_t n_blocks,
                                                         const float4 *__restrict__ x2,
                                                         uint8_t *__restrict__ dst2,
                                                         int32_t n_heads, int64_t head_stride,
                                                         int64_t seq_stride)
{
    const int run = blockIdx.y;
    if (blockIdx.z) {
        x = x2;
        dst = dst2;
    }
    x += (int64_t)run * n_blocks * 8;
    dst += (int64_t)(run / n_heads) * seq_stride + (int64_t)(run % n_heads) * head_stride;
    float4 v[U];
    int64_t blk[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t gid = ((int64_t)blockIdx.x * U + u) * 256 + threadIdx.x;
        blk[u] = gid >> 3;
        // the FP32 source is read once: non-temporal loads keep it from displacing cached data
        floatx4 t = {0.f, 0.f, 0.f, 0.f};
        if (blk[u] < n_blocks)
            t = __builtin_nontemporal_load(reinterpret_cast<const floatx4 *>(x) + gid);
        v[u] = make_float4(t.x, t.y, t.z, t.w);
    }
    const int sub = (int)(threadIdx.x & 7);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float a = fmaxf(fmaxf(fabsf(v[u].x), fabsf(v[u].y)),
                        fmaxf(fabsf(v[u].z), fabsf(v[u].w)));
        // the block's eight lanes: swap neighbours, then pairs, then the two quads (mirror)
        a = fmaxf(a, dpp<kDppQuadSwap1>(a));
        a = fmaxf(a, dpp<kDppQuadSwap2>(a));
        a = fmaxf(a, dpp<kDppHalfMirror>(a));
        const __half d16 = __float2half_rn(div127(a));
        const float dh = __half2float(d16);
        const float rdh = __builtin_amdgcn_rcpf(dh);
        bool near_tie;
        uint32_t q = quantise4_fast(v[u], rdh, near_tie);
        if (near_tie || !(dh >= 0x1p-14f)) { // a value next to a tie, or a zero or subnormal scale
            const int q0 = quantise(v[u].x, dh, rdh), q1 = quantise(v[u].y, dh, rdh);
            const int q2 = quantise(v[u].z, dh, rdh), q3 = quantise(v[u].w, dh, rdh);
            q = (uint32_t)(q0 & 0xff) | (uint32_t)(q1 & 0xff) << 8 | (uint32_t)(q2 & 0xff) << 16 |
                (uint32_t)(q3 & 0xff) << 24;
        }
        if (blk[u] < n_blocks) {
            uint8_t *out = dst + blk[u] * 34;
            // non-temporal stores: streamed out, not kept in the L2 for the end-of-launch
            // write-back
            if (sub == 0)
                __builtin_nontemporal_store(__half_as_ushort(d16),
                                            reinterpret_cast<uint16_t *>(out));
            // the lane's four bytes in one store (2-byte aligned: the hardware takes unaligned
            // dword accesses)
            __builtin_nontemporal_store(q, reinterpret_cast<u32_a2 *>(out + 2 + 4 * sub));
        }
    }
}

} // namespace

constexpr int kPackU = 2; // blocks per lane group of 8 (two 16-byte loads in flight per lane)

hipError_t launch_q8_0_pack(const float *x, uint8_t *dst, int64_t n_blocks, hipStream_t s)
{
    if (n_blocks == 0)
        return hipSuccess;
    const int64_t threads = n_blocks * 8;
    const int64_t grid = (threads + 256 * kPackU - 1) / (256 * kPackU);
    hipLaunchKernelGGL(q8_0_pack_kernel<kPackU>, dim3((unsigned)grid), dim3(256), 0, s,
                       reinterpret_cast<const float4 *>(x), dst, n_blocks,
                       reinterpret_cast<const float4 *>(x), dst, 1, (int64_t)0, (int64_t)0);
    return hipGetLastError();
}

hipError_t launch_q8_0_pack_rows(const float *k, const float *v, uint8_t *k_dst, uint8_t *v_dst,
                                 int32_t n_seq, int32_t n_heads, int32_t n_rows,
                                 int64_t head_stride, int64_t seq_stride, hipStream_t s)
{
    const int64_t n_blocks = (int64_t)n_rows * (kHeadDim / 32); // per (sequence, head) run
    const int64_t grid = (n_blocks * 8 + 256 * kPackU - 1) / (256 * kPackU);
    hipLaunchKernelGGL(q8_0_pack_kernel<kPackU>,
                       dim3((unsigned)grid, (unsigned)(n_seq * n_heads), 2), dim3(256), 0, s,
                       reinterpret_cast<const float4 *>(k), k_dst, n_blocks,
                       reinterpret_cast<const float4 *>(v), v_dst, n_heads, head_stride,
                       seq_stride);
    return hipGetLastError();
}

} // namespace q8a
