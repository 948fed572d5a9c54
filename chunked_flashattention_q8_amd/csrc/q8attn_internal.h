// Internal declarations shared by the translation units of libq8attn.so (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q8a {

constexpr int kHeadDim = 64;
constexpr int kQ8RowBytes = 68;   // two 34-byte Q8_0 blocks per 64-dim head row
constexpr int kF16RowBytes = 128; // 64 FP16 values

// Arguments of one accumulate launch: the chunk of keys [kv_pos0, kv_pos0 + n_kv) of every
// (sequence, head) pair, applied to the state rows of that pair.
struct AccumulateArgs {
    const void *q;          // FP16 [B][H][M][64]
    const uint8_t *k;       // key 0 of sequence 0, head 0
    const uint8_t *v;
    float *m, *l, *o;       // state
    int64_t kv_head_stride; // bytes
    int64_t kv_seq_stride;  // bytes
    int64_t q_pos0;
    int64_t kv_pos0;
    int32_t B, H, M;
    int32_t n_kv;
    int32_t causal;
    // optional: the final output of the rows whose query position lies inside the chunk
    // (null: none); out FP16 [B][H][M][64], lse FP32 [B][H][M] or null
    void *out;
    float *lse;
    // 1: those rows get out/lse only, their m/l/O are not written
    int32_t final_out_only;
    // 1: the state holds nothing yet and every row sees a key of this chunk: no state is read,
    // and every row is written (rows that saw no key as empty)
    int32_t fresh;
    // tile form for more than 64 query rows: kFormAuto (the library's choice) or one forced
    int32_t form;
};

// forced tile forms of the accumulate kernel (AccumulateArgs::form)
constexpr int kFormAuto = 0, kFormWide = 1, kFormNarrow = 2, kFormKeySplit = 3, kFormSplit = 4;

hipError_t launch_q8_0_pack(const float *x, uint8_t *dst, int64_t n_blocks, hipStream_t s);
// K and V rows [n_seq][n_heads][n_rows][64] FP32 -> Q8_0 rows at k_dst / v_dst + b * seq_stride
// + h * head_stride + j * 68 (one launch for both tensors)
hipError_t launch_q8_0_pack_rows(const float *k, const float *v, uint8_t *k_dst, uint8_t *v_dst,
                                 int32_t n_seq, int32_t n_heads, int32_t n_rows,
                                 int64_t head_stride, int64_t seq_stride, hipStream_t s);
hipError_t launch_state_init(float *m, float *l, int64_t n_rows, hipStream_t s);
hipError_t launch_accumulate(const AccumulateArgs &a, int kv_dtype, hipStream_t s);
hipError_t launch_finalize(const float *m, const float *l, const float *o, void *out,
                           float *lse, int64_t n_rows, hipStream_t s);
hipError_t launch_merge(float *ma, float *la, float *oa, const float *mb, const float *lb,
                        const float *ob, int64_t n_rows, hipStream_t s);

} // namespace q8a
