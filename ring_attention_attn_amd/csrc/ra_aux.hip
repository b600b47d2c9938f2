// Bandwidth-bound kernels of the path: the log-sum-exp merge of step partials,
// the backward preprocess D = rowsum(dO * O) (+ bf16 cast of O), the local head
// permute of the head-parallel all-to-all, and a fill. All are HBM-bound: each
// lane moves 16-byte vectors along the contiguous head_dim axis.
#include <limits.h>
#include <math.h>

#include "ra_internal.h"

namespace {

constexpr int kBlock = 256;

inline unsigned grid_for(int64_t work, int64_t per_block, int64_t cap = 1 << 20) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (unsigned)g;
}

// ---------------------------------------------------------------- lse_merge
// One thread per 4 consecutive floats of O; the D/4 threads of one (row, head)
// vector sit in one wave, so every lane reads the old lse_acc before the one
// lane that owns it stores the new value (in-order issue within a wave).
// Only the rows [row_begin, row_begin + row_count) of the [rows][hq][d] tensors
// are touched (the rows a ring step gave any visible key).
template <int D>
__global__ __launch_bounds__(kBlock) void lse_merge_kernel(int64_t rows, int32_t hq,
                                                           int64_t row_begin, int64_t row_count,
                                                           float* __restrict__ o_acc,
                                                           float* __restrict__ lse_acc,
                                                           const float* __restrict__ o_step,
                                                           const float* __restrict__ lse_step) {
  constexpr int TPV = D / 4;  // threads per (row, head) vector
  const int64_t nvec4 = row_count * hq * TPV;
  for (int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x; t < nvec4;
       t += (int64_t)gridDim.x * kBlock) {
    const int64_t vec = row_begin * hq + t / TPV;  // (row, head) pair, row-major
    const int x4 = (int)(t % TPV);
    // (rows * hq < 2^32, checked by the caller: 32-bit division)
    const uint32_t v32 = (uint32_t)vec;
    const int64_t row = (int64_t)(v32 / (uint32_t)hq);
    const int h = (int)(v32 % (uint32_t)hq);
    const int64_t li = (int64_t)h * rows + row;
    const float la = lse_acc[li];
    const float ls = lse_step[li];
    const float m = fmaxf(la, ls);
    if (m == -INFINITY) continue;  // both empty: leave the accumulator as it is
    const float ea = expf(la - m), es = expf(ls - m);
    const float tot = ea + es;
    const float inv = 1.0f / tot;
    const float ca = ea * inv, cs = es * inv;
    // O is streamed once: non-temporal 16-byte loads and stores
    f32x4* oa = reinterpret_cast<f32x4*>(o_acc + vec * D) + x4;
    const f32x4 os =
        __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(o_step + vec * D) + x4);
    f32x4 a = __builtin_nontemporal_load(oa);
    a = ca * a + cs * os;
    __builtin_nontemporal_store(a, oa);
    if (x4 == 0) lse_acc[li] = m + logf(tot);
  }
}

// ---------------------------------------------------------------- bwd delta
// G = D/8 lanes per (row, head) vector, 8 elements per lane, reduced by xor
// shuffles inside the lane group.
template <int D, bool BF16>
__global__ __launch_bounds__(kBlock) void bwd_delta_kernel(int64_t rows, int32_t hq,
                                                           const float* __restrict__ o,
                                                           const void* __restrict__ dout,
                                                           float* __restrict__ delta,
                                                           bf16_t* __restrict__ o_out) {
  constexpr int G = D / 8;
  const int64_t nvec = rows * hq;
  const int64_t total = nvec * G;
  for (int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x; t - (threadIdx.x % G) < total;
       t += (int64_t)gridDim.x * kBlock) {
    const bool valid = t < total;
    const int64_t vec = valid ? t / G : 0;
    const int sub = (int)(t % G);
    float acc = 0.f;
    if (valid) {
      // O and dO are streamed once: non-temporal 16-byte loads (and stores)
      const f32x4* op = reinterpret_cast<const f32x4*>(o + vec * D + sub * 8);
      const f32x4 o0 = __builtin_nontemporal_load(op), o1 = __builtin_nontemporal_load(op + 1);
      float dv[8];
      if (BF16) {
        const bf16x8 g8 = __builtin_nontemporal_load(
            reinterpret_cast<const bf16x8*>((const bf16_t*)dout + vec * D + sub * 8));
#pragma unroll
        for (int e = 0; e < 8; ++e) dv[e] = (float)g8[e];
      } else {
        const f32x4* gp = reinterpret_cast<const f32x4*>((const float*)dout + vec * D + sub * 8);
        const f32x4 g0 = __builtin_nontemporal_load(gp), g1 = __builtin_nontemporal_load(gp + 1);
#pragma unroll
        for (int e = 0; e < 4; ++e) { dv[e] = g0[e]; dv[4 + e] = g1[e]; }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) acc += dv[e] * o0[e] + dv[4 + e] * o1[e];
      if (o_out) {
        bf16x8 ob;
#pragma unroll
        for (int e = 0; e < 4; ++e) { ob[e] = (bf16_t)o0[e]; ob[4 + e] = (bf16_t)o1[e]; }
        __builtin_nontemporal_store(ob, reinterpret_cast<bf16x8*>(o_out + vec * D + sub * 8));
      }
    }
#pragma unroll
    for (int off = G / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, G);
    if (valid && sub == 0) {
      // (rows * hq < 2^32, checked by the caller: 32-bit division)
      const uint32_t v32 = (uint32_t)vec;
      const int64_t row = (int64_t)(v32 / (uint32_t)hq);
      const int h = (int)(v32 % (uint32_t)hq);
      delta[(int64_t)h * rows + row] = acc;
    }
  }
}

// ---------------------------------------------------------------- head permute
// A copy of s*p contiguous runs of run16 16-byte vectors: run (q, t) of the
// [p][s][h/p][d] side is run (t, q) of the [s][h][d] side. Block (x, q) copies
// the runs of group q for tokens x*rpb .. x*rpb + rpb - 1 (rpb = runs per
// block), one vector per thread (runs longer than a block loop), so the index
// arithmetic is a few integer operations per thread; every byte is read and
// written once, with non-temporal hints.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(kBlock) void head_permute_kernel(const i32x4* __restrict__ src,
                                                              i32x4* __restrict__ dst, int64_t s,
                                                              int32_t p, int32_t run16,
                                                              int32_t rpb, int32_t inverse) {
  const int q = blockIdx.y;
  const int lr = rpb > 1 ? (int)threadIdx.x / run16 : 0;
  if (lr >= rpb) return;
  const int64_t tok = (int64_t)blockIdx.x * rpb + lr;
  if (tok >= s) return;
  const int64_t grouped = ((int64_t)q * s + tok) * run16;  // [p][s] side
  const int64_t flat = (tok * p + q) * run16;             // [s][h] side
  const i32x4* from = src + (inverse ? grouped : flat);
  i32x4* to = dst + (inverse ? flat : grouped);
  for (int off = (int)threadIdx.x - lr * run16; off < run16; off += kBlock)
    __builtin_nontemporal_store(__builtin_nontemporal_load(from + off), to + off);
}

__global__ __launch_bounds__(kBlock) void fill_kernel(float* __restrict__ dst, int64_t n, float v) {
  for (int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x; t < n;
       t += (int64_t)gridDim.x * kBlock)
    dst[t] = v;
}

}  // namespace

hipError_t launch_lse_merge(int64_t rows, int32_t hq, int32_t d, int64_t row_begin,
                            int64_t row_count, float* o_acc, float* lse_acc, const float* o_step,
                            const float* lse_step, hipStream_t s) {
  const int64_t work = row_count * hq * (d / 4);
  const unsigned g = grid_for(work, kBlock * 4, 8192);
  if (d == 128)
    hipLaunchKernelGGL(lse_merge_kernel<128>, dim3(g), dim3(kBlock), 0, s, rows, hq, row_begin,
                       row_count, o_acc, lse_acc, o_step, lse_step);
  else
    hipLaunchKernelGGL(lse_merge_kernel<64>, dim3(g), dim3(kBlock), 0, s, rows, hq, row_begin,
                       row_count, o_acc, lse_acc, o_step, lse_step);
  return hipGetLastError();
}

hipError_t launch_bwd_delta(int64_t rows, int32_t hq, int32_t d, int32_t dtype, const float* o,
                            const void* dout, float* delta, void* o_out, hipStream_t s) {
  const int64_t work = rows * hq * (d / 8);
  const unsigned g = grid_for(work, kBlock * 2, 8192);
  bf16_t* ob = (bf16_t*)o_out;
  if (d == 128) {
    if (dtype == RA_BF16)
      hipLaunchKernelGGL((bwd_delta_kernel<128, true>), dim3(g), dim3(kBlock), 0, s, rows, hq, o,
                         dout, delta, ob);
    else
      hipLaunchKernelGGL((bwd_delta_kernel<128, false>), dim3(g), dim3(kBlock), 0, s, rows, hq, o,
                         dout, delta, ob);
  } else {
    if (dtype == RA_BF16)
      hipLaunchKernelGGL((bwd_delta_kernel<64, true>), dim3(g), dim3(kBlock), 0, s, rows, hq, o,
                         dout, delta, ob);
    else
      hipLaunchKernelGGL((bwd_delta_kernel<64, false>), dim3(g), dim3(kBlock), 0, s, rows, hq, o,
                         dout, delta, ob);
  }
  return hipGetLastError();
}

hipError_t launch_head_permute(const void* src, void* dst, int64_t s, int32_t h, int32_t d,
                               int32_t p, int32_t elem_bytes, int32_t inverse, hipStream_t st) {
  const int64_t run16 = (int64_t)(h / p) * d * elem_bytes / 16;
  if (run16 > INT32_MAX) return hipErrorInvalidValue;
  const int32_t rpb = run16 >= kBlock ? 1 : (int32_t)(kBlock / run16);
  const int64_t gx = (s + rpb - 1) / rpb;
  if (gx > INT32_MAX || p > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(head_permute_kernel, dim3((unsigned)gx, (unsigned)p), dim3(kBlock), 0, st,
                     (const i32x4*)src, (i32x4*)dst, s, p, (int32_t)run16, rpb, inverse);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* dst, int64_t n, float value, hipStream_t s) {
  const unsigned g = grid_for(n, kBlock * 16, 16384);
  hipLaunchKernelGGL(fill_kernel, dim3(g), dim3(kBlock), 0, s, dst, n, value);
  return hipGetLastError();
}
