// Backward of one ring step, driven by the final per-row log-sum-exp and
// D = rowsum(dO * O) (saved-LSE recompute): with P = exp(s - LSE),
// dP = dO V^T, dS = P (dP - D): dV += P^T dO, dK += scale dS^T Q,
// dQ += scale dS K; dK/dV sum over the query heads sharing a KV head.
//
// bf16 path (gfx950 MFMA), key-stationary: a workgroup of 4 waves owns 128 keys
// of one KV head (32 per wave, K and V held in registers as MFMA operands) and
// walks the query tiles (64 rows) of every query head of the group. Per tile a
// wave computes S = Q K^T and dP = dO V^T (lanes = keys, registers = queries),
// so P and dS are directly the B operands of dV^T += dO^T P and
// dK^T += Q^T dS, with dO^T and Q^T read from LDS by ds_read_b64_tr_b16. dS is
// also written to LDS (key-major), and the workgroup forms
// dQ_tile = dS K over its 128 keys, added to dq_acc with fp32 atomics.
//
// fp32 path: plain VALU kernels, one per output (dQ row-stationary, dK/dV
// key-stationary), deterministic.
#include <math.h>

#include "ra_internal.h"

namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ inline float to_f(bf16_t x) { return (float)x; }
__device__ inline float to_f(float x) { return x; }

// ============================================================= VALU kernels
template <int D, typename T>
__global__ __launch_bounds__(64) void bwd_dq_simple_kernel(StepParams p) {
  constexpr int TPR = D / 64;
  constexpr int RPB = 64 / TPR;
  constexpr int KT = 32;
  __shared__ float sK[KT][D];
  __shared__ float sV[KT][D];
  const int h = blockIdx.y;
  const int g = h / p.group;
  const int sub = threadIdx.x % TPR;
  const int64_t r0 = (int64_t)blockIdx.x * RPB;
  const int64_t row = r0 + threadIdx.x / TPR;
  const int64_t lq = p.qm.len;
  const bool valid = row < lq;
  const int64_t qpos = valid ? seg_pos(p.qm, row) : -1;
  int64_t qlo, qhi;
  seg_bounds(p.qm, r0, r0 + RPB < lq ? r0 + RPB : lq, qlo, qhi);
  const T* Q = (const T*)p.q;
  const T* K = (const T*)p.k;
  const T* V = (const T*)p.v;
  const T* dO = (const T*)p.dout;
  float q[64], dq[64], go[64];
#pragma unroll
  for (int x = 0; x < 64; ++x) {
    q[x] = valid ? to_f(Q[row * p.q_ss + h * p.q_hs + sub * 64 + x]) : 0.f;
    go[x] = valid ? to_f(dO[row * p.do_ss + h * p.do_hs + sub * 64 + x]) : 0.f;
    dq[x] = 0.f;
  }
  const float lse = valid ? p.lse_in[(int64_t)h * lq + row] : 0.f;
  const float dlt = valid ? p.delta[(int64_t)h * lq + row] : 0.f;
  for (int64_t k0 = 0; k0 < p.km.len; k0 += KT) {
    const int64_t k1 = k0 + KT < p.km.len ? k0 + KT : p.km.len;
    int64_t klo, khi;
    seg_bounds(p.km, k0, k1, klo, khi);
    if (p.causal && klo > qhi) continue;
    __syncthreads();
    for (int i = threadIdx.x; i < KT * D; i += 64) {
      const int kr = i / D, x = i % D;
      const int64_t key = k0 + kr;
      sK[kr][x] = key < k1 ? to_f(K[key * p.k_ss + g * p.k_hs + x]) : 0.f;
      sV[kr][x] = key < k1 ? to_f(V[key * p.v_ss + g * p.v_hs + x]) : 0.f;
    }
    __syncthreads();
    for (int j = 0; j < (int)(k1 - k0); ++j) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int x = 0; x < 64; ++x) {
        s += q[x] * sK[j][sub * 64 + x];
        dp += go[x] * sV[j][sub * 64 + x];
      }
      if (TPR == 2) {
        s += __shfl_xor(s, 1);
        dp += __shfl_xor(dp, 1);
      }
      const int64_t kpos = seg_pos(p.km, k0 + j);
      if (!valid || (p.causal && kpos > qpos) || lse == -INFINITY) continue;
      const float pr = expf(s * p.scale - lse);
      const float ds = pr * (dp - dlt);
#pragma unroll
      for (int x = 0; x < 64; ++x) dq[x] += ds * sK[j][sub * 64 + x];
    }
  }
  if (!valid) return;
#pragma unroll
  for (int x = 0; x < 64; ++x) p.o[row * p.o_ss + h * p.o_hs + sub * 64 + x] += p.scale * dq[x];
}

template <int D, typename T>
__global__ __launch_bounds__(64) void bwd_dkv_simple_kernel(StepParams p) {
  constexpr int TPR = D / 64;
  constexpr int KPB = 64 / TPR;  // keys per block
  constexpr int QTL = 32;
  __shared__ float sQ[QTL][D];
  __shared__ float sO[QTL][D];
  __shared__ float sL[QTL], sDl[QTL];
  __shared__ int64_t sP[QTL];
  const int g = blockIdx.y;
  const int sub = threadIdx.x % TPR;
  const int64_t k0 = (int64_t)blockIdx.x * KPB;
  const int64_t key = k0 + threadIdx.x / TPR;
  const int64_t lk = p.km.len, lq = p.qm.len;
  const bool valid = key < lk;
  const int64_t kpos = valid ? seg_pos(p.km, key) : INT64_MAX;
  int64_t klo, khi;
  seg_bounds(p.km, k0, k0 + KPB < lk ? k0 + KPB : lk, klo, khi);
  const T* Q = (const T*)p.q;
  const T* K = (const T*)p.k;
  const T* V = (const T*)p.v;
  const T* dO = (const T*)p.dout;
  float kk[64], vv[64], dk[64], dv[64];
#pragma unroll
  for (int x = 0; x < 64; ++x) {
    kk[x] = valid ? to_f(K[key * p.k_ss + g * p.k_hs + sub * 64 + x]) : 0.f;
    vv[x] = valid ? to_f(V[key * p.v_ss + g * p.v_hs + sub * 64 + x]) : 0.f;
    dk[x] = 0.f;
    dv[x] = 0.f;
  }
  for (int hh = 0; hh < p.group; ++hh) {
    const int h = g * p.group + hh;
    for (int64_t q0 = 0; q0 < lq; q0 += QTL) {
      const int64_t q1 = q0 + QTL < lq ? q0 + QTL : lq;
      int64_t tlo, thi;
      seg_bounds(p.qm, q0, q1, tlo, thi);
      if (p.causal && thi < klo) continue;
      __syncthreads();
      for (int i = threadIdx.x; i < QTL * D; i += 64) {
        const int qr = i / D, x = i % D;
        const int64_t row = q0 + qr;
        sQ[qr][x] = row < q1 ? to_f(Q[row * p.q_ss + h * p.q_hs + x]) : 0.f;
        sO[qr][x] = row < q1 ? to_f(dO[row * p.do_ss + h * p.do_hs + x]) : 0.f;
      }
      if (threadIdx.x < QTL) {
        const int64_t row = q0 + threadIdx.x;
        sL[threadIdx.x] = row < q1 ? p.lse_in[(int64_t)h * lq + row] : -INFINITY;
        sDl[threadIdx.x] = row < q1 ? p.delta[(int64_t)h * lq + row] : 0.f;
        sP[threadIdx.x] = row < q1 ? seg_pos(p.qm, row) : -1;
      }
      __syncthreads();
      for (int i = 0; i < (int)(q1 - q0); ++i) {
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int x = 0; x < 64; ++x) {
          s += kk[x] * sQ[i][sub * 64 + x];
          dp += vv[x] * sO[i][sub * 64 + x];
        }
        if (TPR == 2) {
          s += __shfl_xor(s, 1);
          dp += __shfl_xor(dp, 1);
        }
        if (!valid || (p.causal && kpos > sP[i]) || sL[i] == -INFINITY) continue;
        const float pr = expf(s * p.scale - sL[i]);
        const float ds = pr * (dp - sDl[i]);
#pragma unroll
        for (int x = 0; x < 64; ++x) {
          dv[x] += pr * sO[i][sub * 64 + x];
          dk[x] += ds * sQ[i][sub * 64 + x];
        }
      }
    }
  }
  if (!valid) return;
  float* dkp = p.dk + key * p.dk_ss + (int64_t)g * p.dk_hs + sub * 64;
  float* dvp = p.dv + key * p.dk_ss + (int64_t)g * p.dk_hs + sub * 64;
#pragma unroll
  for (int x = 0; x < 64; ++x) {
    const float a = p.scale * dk[x], b = dv[x];
    dkp[x] = p.dkv_accumulate ? dkp[x] + a : a;
    dvp[x] = p.dkv_accumulate ? dvp[x] + b : b;
  }
}

// ============================================================= MFMA kernel
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ inline bf16x4 ds_read_tr(const bf16_t* lds_ptr) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_ptr));
  return __builtin_bit_cast(bf16x4, r);
}

// A 32x16 (or 16x32) MFMA operand slice whose 8 contraction values per lane
// come from 4+4 consecutive LDS rows at one column: rows base_row + tr_row and
// base_row + 8 + tr_row, column base_col + tr_col (lane roles precomputed).
__device__ inline bf16x8 tr_operand(const bf16_t* lds, int stride, int row, int col) {
  const bf16x4 a = ds_read_tr(lds + row * stride + col);
  const bf16x4 b = ds_read_tr(lds + (row + 8) * stride + col);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int D>
__global__ __launch_bounds__(256, 1) void bwd_mfma_kernel(StepParams p, int n_kt) {
  constexpr int KB = 128;         // keys per workgroup, 32 per wave
  constexpr int QT = 64;          // query rows per iteration (two 32-row blocks)
  constexpr int NC = D / 16;
  constexpr int ND = D / 32;
  constexpr int NDW = ND / 2;     // dQ d-blocks per wave
  constexpr int QSTR = D + 16;    // LDS strides (elements)
  constexpr int KSTR = D + 16;
  constexpr int SSTR = QT + 16;
  constexpr int CPR = D / 8;      // 16-byte chunks per row
  constexpr int NLQ = QT * CPR / 256;
  constexpr int NLK = KB * CPR / 256;
  __shared__ __attribute__((aligned(16))) bf16_t sQ[QT * QSTR];
  __shared__ __attribute__((aligned(16))) bf16_t sdO[QT * QSTR];
  __shared__ __attribute__((aligned(16))) bf16_t sK[KB * KSTR];
  __shared__ __attribute__((aligned(16))) bf16_t sdsT[KB * SSTR];
  __shared__ float sL[QT], sDl[QT];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int grp = lane >> 4, gi = lane & 15;
  const int tr_row = 4 * (grp >> 1) + (gi >> 2);
  const int tr_col = 16 * (grp & 1) + 4 * (gi & 3);

  const int total = p.hkv * n_kt;
  const int w = blockIdx.x;
  const int logical = (total % 8 == 0) ? (w % 8) * (total / 8) + (w / 8) : w;
  const int g = logical / n_kt;
  const int kt = logical % n_kt;  // earlier keys (seen by more queries) first
  const int64_t lq = p.qm.len, lk = p.km.len;
  const int64_t key0 = (int64_t)kt * KB;
  const int64_t key1 = key0 + KB < lk ? key0 + KB : lk;
  const int64_t wkey0 = key0 + wave * 32;
  const int64_t mykey = wkey0 + l32;
  const bool key_ok = mykey < lk;
  const int64_t kpos = key_ok ? seg_pos(p.km, mykey) : INT64_MAX;
  int64_t gk_lo, gk_hi, wk_lo = INT64_MAX, wk_hi = INT64_MIN;
  seg_bounds(p.km, key0, key1, gk_lo, gk_hi);
  const bool wave_has_keys = wkey0 < lk;
  if (wave_has_keys) seg_bounds(p.km, wkey0, wkey0 + 32 < lk ? wkey0 + 32 : lk, wk_lo, wk_hi);

  const bf16_t* Kg = (const bf16_t*)p.k + (int64_t)g * p.k_hs;
  const bf16_t* Vg = (const bf16_t*)p.v + (int64_t)g * p.v_hs;

  // K^T / V^T as B operands: lane = key column, d = 16c + 8*hi .. +8
  bf16x8 kreg[NC], vreg[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    bf16x8 z = {};
    kreg[c] = key_ok ? *(const bf16x8*)(Kg + mykey * p.k_ss + 16 * c + 8 * hi) : z;
    vreg[c] = key_ok ? *(const bf16x8*)(Vg + mykey * p.v_ss + 16 * c + 8 * hi) : z;
  }
  // K tile in LDS (row-major) for dQ = dS K
#pragma unroll
  for (int i = 0; i < NLK; ++i) {
    const int c = i * 256 + tid;
    const int r = c / CPR, col = (c % CPR) * 8;
    const int64_t key = key0 + r;
    bf16x8 z = {};
    *(bf16x8*)(sK + r * KSTR + col) = key < lk ? *(const bf16x8*)(Kg + key * p.k_ss + col) : z;
  }

  f32x16 dkacc[ND], dvacc[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) {
    dkacc[db] = f32x16{};
    dvacc[db] = f32x16{};
  }

  const int n_qt = (int)((lq + QT - 1) / QT);
  const int n_it = p.group * n_qt;  // (head, query tile) iterations
  auto tile_bounds = [&](int it, int64_t& lo, int64_t& hi_) {
    const int64_t q0 = (int64_t)(it % n_qt) * QT;
    seg_bounds(p.qm, q0, q0 + QT < lq ? q0 + QT : lq, lo, hi_);
  };
  auto next_visible = [&](int it) {
    while (it < n_it) {
      if (!p.causal) return it;
      int64_t lo, hh;
      tile_bounds(it, lo, hh);
      if (hh >= gk_lo) return it;
      ++it;
    }
    return it;
  };

  bf16x8 qr[NLQ], dr[NLQ];
  auto load_regs = [&](int it) {
    const int h = g * p.group + it / n_qt;
    const int64_t q0 = (int64_t)(it % n_qt) * QT;
    const bf16_t* Qh = (const bf16_t*)p.q + (int64_t)h * p.q_hs;
    const bf16_t* Dh = (const bf16_t*)p.dout + (int64_t)h * p.do_hs;
#pragma unroll
    for (int i = 0; i < NLQ; ++i) {
      const int c = i * 256 + tid;
      const int r = c / CPR, col = (c % CPR) * 8;
      const int64_t row = q0 + r;
      bf16x8 z = {};
      qr[i] = row < lq ? *(const bf16x8*)(Qh + row * p.q_ss + col) : z;
      dr[i] = row < lq ? *(const bf16x8*)(Dh + row * p.do_ss + col) : z;
    }
  };

  int it = p.hkv > 0 && lq > 0 ? next_visible(0) : n_it;
  if (it < n_it) load_regs(it);
  while (it < n_it) {
    const int h = g * p.group + it / n_qt;
    const int64_t q0 = (int64_t)(it % n_qt) * QT;
    __syncthreads();  // previous iteration finished with sQ, sdO, sdsT, sL
#pragma unroll
    for (int i = 0; i < NLQ; ++i) {
      const int c = i * 256 + tid;
      const int r = c / CPR, col = (c % CPR) * 8;
      *(bf16x8*)(sQ + r * QSTR + col) = qr[i];
      *(bf16x8*)(sdO + r * QSTR + col) = dr[i];
    }
    if (tid < QT) {
      const int64_t row = q0 + tid;
      float l2 = INFINITY, dl = 0.f;
      if (row < lq) {
        const float lse = p.lse_in[(int64_t)h * lq + row];
        l2 = lse == -INFINITY ? INFINITY : lse * kLog2e;  // empty row: no contribution
        dl = p.delta[(int64_t)h * lq + row];
      }
      sL[tid] = l2;
      sDl[tid] = dl;
    }
    __syncthreads();
    const int itn = next_visible(it + 1);
    if (itn < n_it) load_regs(itn);

    int64_t tq_lo, tq_hi;
    tile_bounds(it, tq_lo, tq_hi);
    const bool wave_skip = !wave_has_keys || (p.causal && tq_hi < wk_lo);
    if (wave_skip) {
      // no visible pair for this wave's keys: its dS columns are zero
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bf16x4 z = {};
          *(bf16x4*)(sdsT + (wave * 32 + l32) * SSTR + qb * 32 + 8 * i + 4 * hi) = z;
        }
    } else {
      const bool need_mask = !key_ok || (int64_t)(q0 + QT) > lq || (p.causal && wk_hi > tq_lo) ||
                             (wkey0 + 32 > lk);
      f32x16 sacc[2], pacc[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        sacc[qb] = f32x16{};
        pacc[qb] = f32x16{};
      }
#pragma unroll
      for (int c = 0; c < NC; ++c) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const bf16x8 aq = *(const bf16x8*)(sQ + (qb * 32 + l32) * QSTR + 16 * c + 8 * hi);
          const bf16x8 ao = *(const bf16x8*)(sdO + (qb * 32 + l32) * QSTR + 16 * c + 8 * hi);
          sacc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, kreg[c], sacc[qb], 0, 0, 0);
          pacc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao, vreg[c], pacc[qb], 0, 0, 0);
        }
      }
      // P and dS (lanes = keys, registers = queries 8*(r/4) + 4*hi + r%4)
      bf16x8 pP[2][2], pS[2][2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int qrow = qb * 32 + 8 * i + 4 * hi;
          const f32x4 l4 = *(const f32x4*)(sL + qrow);
          const f32x4 d4 = *(const f32x4*)(sDl + qrow);
          bf16x4 ds4;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r = 4 * i + j;
            float pr = __builtin_amdgcn_exp2f(sacc[qb][r] * p.scale_log2 - l4[j]);
            if (need_mask) {
              const int64_t row = q0 + qrow + j;
              const bool vis = key_ok && row < lq && (!p.causal || kpos <= seg_pos(p.qm, row));
              pr = vis ? pr : 0.f;
            }
            const float ds = pr * (pacc[qb][r] - d4[j]);
            pP[qb][i >> 1][(i & 1) * 4 + j] = (bf16_t)pr;
            const bf16_t dsb = (bf16_t)ds;
            pS[qb][i >> 1][(i & 1) * 4 + j] = dsb;
            ds4[j] = dsb;
          }
          *(bf16x4*)(sdsT + (wave * 32 + l32) * SSTR + qrow) = ds4;
        }
      }
      // dV^T += dO^T P, dK^T += Q^T dS (contraction over the 64 queries)
#pragma unroll
      for (int db = 0; db < ND; ++db) {
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const bf16x8 ao = tr_operand(sdO, QSTR, 16 * cc + tr_row, 32 * db + tr_col);
          dvacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao, pP[cc >> 1][cc & 1], dvacc[db], 0, 0, 0);
          const bf16x8 aq = tr_operand(sQ, QSTR, 16 * cc + tr_row, 32 * db + tr_col);
          dkacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, pS[cc >> 1][cc & 1], dkacc[db], 0, 0, 0);
        }
      }
    }
    __syncthreads();  // all dS columns in LDS
    // dQ tile = dS (64 q x 128 keys) K (128 keys x D); wave -> (query block, d blocks)
    {
      const int qb = wave >> 1;
      f32x16 qacc[NDW];
#pragma unroll
      for (int j = 0; j < NDW; ++j) qacc[j] = f32x16{};
      const int kc_end = (int)((key1 - key0 + 15) / 16);
      for (int kc = 0; kc < kc_end; ++kc) {
        const bf16x8 a = tr_operand(sdsT, SSTR, 16 * kc + tr_row, qb * 32 + tr_col);
#pragma unroll
        for (int j = 0; j < NDW; ++j) {
          const int db = (wave & 1) * NDW + j;
          const bf16x8 b = tr_operand(sK, KSTR, 16 * kc + tr_row, 32 * db + tr_col);
          qacc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, qacc[j], 0, 0, 0);
        }
      }
#pragma unroll
      for (int j = 0; j < NDW; ++j) {
        const int db = (wave & 1) * NDW + j;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = q0 + qb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (row < lq)
            unsafeAtomicAdd(p.o + row * p.o_ss + (int64_t)h * p.o_hs + 32 * db + l32,
                            qacc[j][r] * p.scale);
        }
      }
    }
    it = itn;
  }

  // ---- epilogue: lanes = keys, registers = d rows 8*(r/4) + 4*hi + r%4
  if (!key_ok) return;
  float* dkp = p.dk + mykey * p.dk_ss + (int64_t)g * p.dk_hs;
  float* dvp = p.dv + mykey * p.dk_ss + (int64_t)g * p.dk_hs;
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4 a, b;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a[j] = dkacc[db][4 * i + j] * p.scale;
        b[j] = dvacc[db][4 * i + j];
      }
      f32x4* pa = (f32x4*)(dkp + 32 * db + 8 * i + 4 * hi);
      f32x4* pb = (f32x4*)(dvp + 32 * db + 8 * i + 4 * hi);
      if (p.dkv_accumulate) {
        a += *pa;
        b += *pb;
      }
      *pa = a;
      *pb = b;
    }
}

template <int D, typename T>
hipError_t launch_simple(const StepParams& p, hipStream_t s) {
  constexpr int RPB = 64 / (D / 64);
  if (p.qm.len > 0) {
    const unsigned gx = (unsigned)((p.qm.len + RPB - 1) / RPB);
    hipLaunchKernelGGL((bwd_dq_simple_kernel<D, T>), dim3(gx, p.hq), dim3(64), 0, s, p);
  }
  const unsigned gk = (unsigned)((p.km.len + RPB - 1) / RPB);
  hipLaunchKernelGGL((bwd_dkv_simple_kernel<D, T>), dim3(gk, p.hkv), dim3(64), 0, s, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_mfma(const StepParams& p, hipStream_t s) {
  const int n_kt = (int)((p.km.len + 127) / 128);
  const int64_t grid = (int64_t)p.hkv * n_kt;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((bwd_mfma_kernel<D>), dim3((unsigned)grid), dim3(256), 0, s, p, n_kt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_step_bwd(const StepParams& p, int dtype, int head_dim, hipStream_t s) {
  if (dtype == RA_BF16) return head_dim == 128 ? launch_mfma<128>(p, s) : launch_mfma<64>(p, s);
  return head_dim == 128 ? launch_simple<128, float>(p, s) : launch_simple<64, float>(p, s);
}
