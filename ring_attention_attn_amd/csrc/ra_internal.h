// Internal declarations shared by the HIP translation units of libringattn.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ring_attn.h"

typedef __bf16 bf16_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

// Rows of a query or KV buffer: up to two runs of consecutive global positions.
struct SegMap {
  int64_t pos0, pos1;  // global position of row 0 of each run
  int64_t seg_len;     // rows in run 0 (run 1 holds the rest)
  int64_t len;         // total rows
};

__host__ __device__ inline int64_t seg_pos(const SegMap& m, int64_t i) {
  return i < m.seg_len ? m.pos0 + i : m.pos1 + (i - m.seg_len);
}

// min / max position over rows [r0, r1) (r0 < r1 <= len)
__host__ __device__ inline void seg_bounds(const SegMap& m, int64_t r0, int64_t r1, int64_t& lo,
                                           int64_t& hi) {
  if (r1 <= m.seg_len || r0 >= m.seg_len) {
    lo = seg_pos(m, r0);
    hi = seg_pos(m, r1 - 1);
  } else {
    int64_t a0 = seg_pos(m, r0), a1 = seg_pos(m, m.seg_len - 1);
    int64_t b0 = seg_pos(m, m.seg_len), b1 = seg_pos(m, r1 - 1);
    lo = a0 < b0 ? a0 : b0;
    hi = a1 > b1 ? a1 : b1;
  }
}

struct StepParams {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* lse_in;   // bwd: final LSE [hq][lq]
  const float* delta;    // bwd: D [hq][lq]
  float* o;              // fwd: o_step; bwd: dq_acc
  float* lse_out;        // fwd: lse_step
  float* dk;
  float* dv;
  int64_t q_ss, q_hs, k_ss, k_hs, v_ss, v_hs, o_ss, o_hs, do_ss, do_hs, dk_ss, dk_hs;
  SegMap qm, km;
  int32_t hq, hkv, group;  // group = hq / hkv
  int32_t causal;
  int32_t dkv_accumulate;
  int32_t merge;           // fwd: fold the step into (o, lse_out) = (O_acc, LSE_acc)
  float scale;             // softmax scale
  float scale_log2;        // scale * log2(e)
};

// The key-side inputs of every ring step, for the calls that run the whole
// ring in one launch (bf16 only); the query side and the strides are the
// StepParams'. Passed by value as a kernel argument.
constexpr int kMaxChunks = RA_MAX_CHUNKS;
struct ChunkSet {
  int32_t n;
  const void* k[kMaxChunks];
  const void* v[kMaxChunks];
  SegMap km[kMaxChunks];
};

// kernel launchers (return hipSuccess or the launch error)
hipError_t launch_step_fwd(const StepParams& p, int dtype, int head_dim, hipStream_t s);
hipError_t launch_step_bwd(const StepParams& p, int dtype, int head_dim, hipStream_t s);
hipError_t launch_fwd_chunks(const StepParams& p, const ChunkSet& ch, int head_dim,
                             hipStream_t s);
// dQ of all chunks in one launch (written), then dK/dV of each chunk (p's
// dk/dv strides and dkv_accumulate; dk[i], dv[i] chunk i's outputs)
hipError_t launch_bwd_chunks(const StepParams& p, const ChunkSet& ch, float* const* dk,
                             float* const* dv, const int32_t* dkv_accumulate, int head_dim,
                             hipStream_t s);
hipError_t launch_lse_merge(int64_t rows, int32_t hq, int32_t d, int64_t row_begin,
                            int64_t row_count, float* o_acc, float* lse_acc, const float* o_step,
                            const float* lse_step, hipStream_t s);
hipError_t launch_bwd_delta(int64_t rows, int32_t hq, int32_t d, int32_t dtype, const float* o,
                            const void* dout, float* delta, void* o_out, hipStream_t s);
hipError_t launch_head_permute(const void* src, void* dst, int64_t s, int32_t h, int32_t d,
                               int32_t p, int32_t elem_bytes, int32_t inverse, hipStream_t st);
hipError_t launch_fill_f32(float* dst, int64_t n, float value, hipStream_t s);
