// Backward of one ring step, driven by the final per-row log-sum-exp and
// D = rowsum(dO * O) (saved-LSE recompute): with P = exp(s - LSE),
// dP = dO V^T, dS = P (dP - D): dV += P^T dO, dK += scale dS^T Q,
// dQ += scale dS K; dK/dV sum over the query heads sharing a KV head.
//
// bf16 path (gfx950 MFMA): two deterministic kernels, one per output side
// (described at each kernel): a query-stationary dQ kernel and a
// key-stationary dK/dV kernel. The dQ kernel recomputes S and dP instead of
// exchanging dS through memory, which trades two extra products for no
// atomics and two waves per SIMD.
//
// fp32 path: plain VALU kernels, one per output (dQ row-stationary, dK/dV
// key-stationary), deterministic.
#include <limits.h>
#include <math.h>

#include <type_traits>

#include "ra_internal.h"
#include "ra_tile.h"

// minimum resident workgroups per CU of the dQ kernel
#ifndef RA_BWD_DQ_MINB
#define RA_BWD_DQ_MINB 2
#endif
// 1: transposed operand tiles staged in LDS; 0: read with ds_read_b64_tr_b16
#ifndef RA_BWD_KTT
#define RA_BWD_KTT 0
#endif
#ifndef RA_BWD_QTT
#define RA_BWD_QTT 0
#endif
// 1: dK/dV kernel reads its K^T/V^T operands from LDS instead of registers
#ifndef RA_BWD_KVL
#define RA_BWD_KVL 0
#endif

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

// ============================================================= MFMA kernels
// Operand A of a product that contracts over rows of a tile held row-major in
// LDS (K for dQ^T += K^T dS^T; Q, dO for dK^T, dV^T): 8 values per lane from
// rows base + 8*hi + 0..7 at column col0 + l32 -- either one 16-byte read of a
// transposed copy (TRANSPOSED) or two transposing reads of the row-major tile.
template <bool TRANSPOSED, int RSTR, int TSTR>
__device__ __forceinline__ bf16x8 rows_operand(const bf16_t* rows_tile, const bf16_t* cols_tile,
                                               int base, int col0, int lane) {
  const int l32 = lane & 31, hi = lane >> 5;
  if (TRANSPOSED) return *(const bf16x8*)(cols_tile + (col0 + l32) * TSTR + base + 8 * hi);
  const int grp = lane >> 4, gi = lane & 15;
  const bf16_t* b = rows_tile + (base + 8 * hi + (gi >> 2)) * RSTR + col0 + 16 * (grp & 1) + 4 * (gi & 3);
  const bf16x4 lo4 = ds_read_tr(b);
  const bf16x4 hi4 = ds_read_tr(b + 4 * RSTR);
  return __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
}

// (1) dQ, query-stationary: a workgroup of 8 waves (two per SIMD) shares each
//     64-key K/V tile (LDS-DMA, double-buffered, one barrier per tile); a wave
//     owns 32 query rows of one head. S^T = K Q^T and dP^T = V dO^T put a query
//     in each lane, so LSE and D are per-lane scalars; dS^T (bf16, 8
//     consecutive keys per register chunk thanks to the sigma row order) is the
//     B operand of dQ^T += K^T dS^T, whose A operand is read transposed from
//     the row-major K tile. K rows have a stride of 19 16-byte chunks (b128
//     reads conflict-free, transposing reads nearly so), V rows 17. dq_acc is
//     read-modify-written once per row at the end: no atomics.
template <int D>
__global__ __launch_bounds__(512, 1) void bwd_dq_kernel(StepParams p, int hpw, int n_qt,
                                                        int rows_per_wg) {
  constexpr int NW = 8;
  constexpr int KT = 64;
  constexpr int KSTR = D + 24;   // 19 (D=128) / 11 (D=64) chunks
  constexpr int VSTR = D + 8;    // 17 / 9 chunks
  constexpr int NC = D / 16;
  constexpr int ND = D / 32;
  __shared__ __attribute__((aligned(1024))) bf16_t sK0[KT * KSTR];
  __shared__ __attribute__((aligned(1024))) bf16_t sK1[KT * KSTR];
  __shared__ __attribute__((aligned(1024))) bf16_t sV0[KT * VSTR];
  __shared__ __attribute__((aligned(1024))) bf16_t sV1[KT * VSTR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int l32 = lane & 31, hi = lane >> 5;
  const int srow = sigma32(l32);

  const int nsub = p.group / hpw;
  const int total = p.hkv * nsub * n_qt;
  const int logical = xcd_remap(blockIdx.x, total);
  const int gh = logical / n_qt;
  const int qt = n_qt - 1 - (logical % n_qt);
  const int g = gh / nsub, hs = gh % nsub;
  const int h = g * p.group + hs * hpw + (wave % hpw);
  const int64_t lq = p.qm.len, lk = p.km.len;
  const int64_t wg_r0 = (int64_t)qt * rows_per_wg;
  const int64_t row0 = wg_r0 + (int64_t)(wave / hpw) * 32;

  int64_t wq_lo = 0, wq_hi = -1, gq_lo, gq_hi;
  const bool wave_active = row0 < lq;
  if (wave_active) seg_bounds(p.qm, row0, row0 + 32 < lq ? row0 + 32 : lq, wq_lo, wq_hi);
  seg_bounds(p.qm, wg_r0, wg_r0 + rows_per_wg < lq ? wg_r0 + rows_per_wg : lq, gq_lo, gq_hi);

  const bf16_t* K = (const bf16_t*)p.k + (int64_t)g * p.k_hs;
  const bf16_t* V = (const bf16_t*)p.v + (int64_t)g * p.v_hs;

  // stale LDS must hold finite values (0 * NaN would poison dQ)
  for (int i = tid; i < KT * KSTR / 8; i += NW * 64) {
    ((bf16x8*)sK0)[i] = bf16x8{};
    ((bf16x8*)sK1)[i] = bf16x8{};
  }
  for (int i = tid; i < KT * VSTR / 8; i += NW * 64) {
    ((bf16x8*)sV0)[i] = bf16x8{};
    ((bf16x8*)sV1)[i] = bf16x8{};
  }

  const int64_t qrow = row0 + l32;
  const bool qok = qrow < lq;
  const int qpos = qok ? (int)seg_pos(p.qm, qrow) : -1;
  const int qlim = (p.causal || !qok) ? qpos : INT_MAX;  // last visible key position
  bf16x8 qreg[NC], doreg[NC];
  {
    const bf16_t* Q = (const bf16_t*)p.q + qrow * p.q_ss + (int64_t)h * p.q_hs + 8 * hi;
    const bf16_t* G = (const bf16_t*)p.dout + qrow * p.do_ss + (int64_t)h * p.do_hs + 8 * hi;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      bf16x8 z = {};
      qreg[c] = qok ? *(const bf16x8*)(Q + 16 * c) : z;
      doreg[c] = qok ? *(const bf16x8*)(G + 16 * c) : z;
    }
  }
  float lse2 = INFINITY, dl = 0.f;  // invalid or empty rows: P = 0
  if (qok) {
    const float lse = p.lse_in[(int64_t)h * lq + qrow];
    lse2 = lse == -INFINITY ? INFINITY : lse * kLog2e;
    dl = p.delta[(int64_t)h * lq + qrow];
  }

  f32x16 qacc[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) qacc[db] = f32x16{};

  const KeyTiles<KT> kt_wg(p.km, p.causal, gq_lo, gq_hi);
  const KeyTiles<KT> kt_w(p.km, p.causal, wq_lo, wq_hi);
  const int n_kt = kt_wg.n;

  DmaStage<KT, D, KSTR * 2, NW> kst;
  DmaStage<KT, D, VSTR * 2, NW> vst;
  kst.init(p.k_ss, wave, lane);
  vst.init(p.v_ss, wave, lane);
  auto stage = [&](int t, auto b) {
    constexpr int B = decltype(b)::value;
    kst.issue(K, p.k_ss, (int64_t)t * KT, lk, B ? sK1 : sK0);
    vst.issue(V, p.v_ss, (int64_t)t * KT, lk, B ? sV1 : sV0);
  };

  const int k_lane = srow * KSTR + 8 * hi;
  const int v_lane = srow * VSTR + 8 * hi;
  const int grp = lane >> 4, gi = lane & 15;
  const int kt_lane = (8 * hi + (gi >> 2)) * KSTR + 16 * (grp & 1) + 4 * (gi & 3);

  auto compute = [&](int t, auto b) {
    constexpr int B = decltype(b)::value;
    if (!wave_active) return;
    const bf16_t* cK = (B ? sK1 : sK0);
    const bf16_t* cV = (B ? sV1 : sV0);
    // S^T = K Q^T and dP^T = V dO^T; register r of key block kb is key
    // t*KT + kb*32 + 16*(r/8) + 8*hi + r%8
    f32x16 sacc[2] = {f32x16{}, f32x16{}}, pacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = mfma32(*(const bf16x8*)(cK + k_lane + kb * 32 * KSTR + 16 * c), qreg[c], sacc[kb]);
        pacc[kb] = mfma32(*(const bf16x8*)(cV + v_lane + kb * 32 * VSTR + 16 * c), doreg[c], pacc[kb]);
      }
    if (!kt_w.mask_free(t)) {  // wave-uniform: one branch around branch-free code
      const TileRows tk(p.km, (int64_t)t * KT, KT);
      const MaskBounds mb(tk, qlim, 8 * hi, p.causal);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const bool vis = mb.key_visible(kb * 32 + 16 * (r >> 3) + (r & 7));
          sacc[kb][r] = vis ? sacc[kb][r] : -INFINITY;
        }
    }
    // dS = P (dP - D), P = exp2(S scale_log2 - LSE log2e), rounded to bf16
    bf16x8 dsk[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * hf + e;
          const float pr = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], p.scale_log2, -lse2));
          v[e] = pr * (pacc[kb][r] - dl);
        }
        dsk[kb][hf] = pack_bf16x8(v);
      }
    // dQ^T += K^T dS^T: K^T operand = keys 16*cc + 8*hi .. +8 of d row
    // 32*db + l32, read transposed; consecutive MFMAs use different accumulators
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        const bf16_t* a = cK + kt_lane + 16 * cc * KSTR + 32 * db;
        const bf16x4 lo4 = ds_read_tr(a);
        const bf16x4 hi4 = ds_read_tr(a + 4 * KSTR);
        const bf16x8 ak = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
        qacc[db] = mfma32(ak, dsk[cc >> 1][cc & 1], qacc[db]);
      }
  };

  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  __syncthreads();  // zero-fill done before any DMA lands
  int t = kt_wg.next(0);
  if (t < n_kt) stage(t, B0{});
  // tiles alternate between two buffers; unrolled so each is a distinct array
  while (t < n_kt) {
    wait_vmem();
    __syncthreads();  // tile t visible in buffer 0; every wave is done with buffer 1
    int tn = kt_wg.next(t + 1);
    if (tn < n_kt) stage(tn, B1{});
    compute(t, B0{});
    t = tn;
    if (t >= n_kt) break;
    wait_vmem();
    __syncthreads();
    tn = kt_wg.next(t + 1);
    if (tn < n_kt) stage(tn, B0{});
    compute(t, B1{});
    t = tn;
  }

  if (!qok) return;
  float* dq = p.o + qrow * p.o_ss + (int64_t)h * p.o_hs;
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4* ptr = (f32x4*)(dq + 32 * db + 8 * i + 4 * hi);
      f32x4 v4 = *ptr;
#pragma unroll
      for (int j = 0; j < 4; ++j) v4[j] += qacc[db][4 * i + j] * p.scale;
      *ptr = v4;
    }
}

// (2) dK, dV, key-stationary: a workgroup of 4 waves owns 128 keys of one KV
//     head (32 per wave; K^T and V^T B operands held in registers) and walks the
//     64-row query tiles of every query head of the group. S = Q K^T and
//     dP = dO V^T put a key in each lane (query rows fed in sigma order), so P
//     and dS, rounded to bf16, are directly the B operands of dV^T += dO^T P and
//     dK^T += Q^T dS. Each dK/dV element has one writer.
template <int D, bool QTT, bool KVL>
__global__ __launch_bounds__(256, 1) void bwd_dkv_kernel(StepParams p, int n_kt) {
  constexpr int KB = 128;
  constexpr int QT = 64;
  constexpr int QSTR = D + 16;
  constexpr int QTSTR = QT + 8;
  constexpr int NC = D / 16;
  constexpr int ND = D / 32;
  __shared__ __attribute__((aligned(16))) bf16_t sQ[QT * QSTR];
  __shared__ __attribute__((aligned(16))) bf16_t sdO[QT * QSTR];
  __shared__ __attribute__((aligned(16))) bf16_t sQt[QTT ? D * QTSTR : 8];
  __shared__ __attribute__((aligned(16))) bf16_t sdOt[QTT ? D * QTSTR : 8];
  __shared__ __attribute__((aligned(16))) float sL[QT];
  __shared__ __attribute__((aligned(16))) float sDl[QT];
  // KVL: the workgroup's 128 keys of K and V stay in LDS (row-major) and the
  // B operands are read per use, which keeps vector registers free for
  // in-flight operand loads
  constexpr int KVSTR = D + 8;
  __shared__ __attribute__((aligned(16))) bf16_t sKk[KVL ? KB * KVSTR : 8];
  __shared__ __attribute__((aligned(16))) bf16_t sVv[KVL ? KB * KVSTR : 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int l32 = lane & 31, hi = lane >> 5;
  const int srow = sigma32(l32);

  const int logical = xcd_remap(blockIdx.x, p.hkv * n_kt);
  const int g = logical / n_kt;
  const int kt = logical % n_kt;  // earlier keys (seen by more queries) first
  const int64_t lq = p.qm.len, lk = p.km.len;
  const int64_t key0 = (int64_t)kt * KB;
  const int64_t key1 = key0 + KB < lk ? key0 + KB : lk;
  const int64_t wkey0 = key0 + wave * 32;
  const int64_t mykey = wkey0 + l32;
  const bool key_ok = mykey < lk;
  // first query position that sees this lane's key (never, for a missing key)
  const int kmin = !key_ok ? INT_MAX : (p.causal ? (int)seg_pos(p.km, mykey) : INT_MIN);
  int64_t gk_lo, gk_hi, wk_lo = INT64_MAX, wk_hi = INT64_MIN;
  seg_bounds(p.km, key0, key1, gk_lo, gk_hi);
  const bool wave_has_keys = wkey0 < lk;
  if (wave_has_keys) seg_bounds(p.km, wkey0, wkey0 + 32 < lk ? wkey0 + 32 : lk, wk_lo, wk_hi);

  bf16x8 kreg[KVL ? 1 : NC], vreg[KVL ? 1 : NC];
  if (KVL) {
    RowStage<KB, D, KVSTR> kst, vst;
    kst.init(p.k_ss, tid);
    vst.init(p.v_ss, tid);
    kst.load((const bf16_t*)p.k + (int64_t)g * p.k_hs, p.k_ss, key0, lk);
    vst.load((const bf16_t*)p.v + (int64_t)g * p.v_hs, p.v_ss, key0, lk);
    kst.store(sKk);
    vst.store(sVv);
  } else {
    const bf16_t* Kp = (const bf16_t*)p.k + (int64_t)g * p.k_hs + mykey * p.k_ss + 8 * hi;
    const bf16_t* Vp = (const bf16_t*)p.v + (int64_t)g * p.v_hs + mykey * p.v_ss + 8 * hi;
#pragma unroll
    for (int c = 0; c < (KVL ? 1 : NC); ++c) {
      bf16x8 z = {};
      kreg[c] = key_ok ? *(const bf16x8*)(Kp + 16 * c) : z;
      vreg[c] = key_ok ? *(const bf16x8*)(Vp + 16 * c) : z;
    }
  }
  const bf16_t* kop = sKk + (wave * 32 + l32) * KVSTR + 8 * hi;  // B operand rows (KVL)
  const bf16_t* vop = sVv + (wave * 32 + l32) * KVSTR + 8 * hi;
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

  RowStage<QT, D, QSTR> qs, ds;
  ColStage<QT, D, QTSTR> qts, dts;
  qs.init(p.q_ss, tid);
  ds.init(p.do_ss, tid);
  if (QTT) {
    qts.init(p.q_ss, tid);
    dts.init(p.do_ss, tid);
  }
  auto load = [&](int it) {
    const int h = g * p.group + it / n_qt;
    const int64_t q0 = (int64_t)(it % n_qt) * QT;
    const bf16_t* Qh = (const bf16_t*)p.q + (int64_t)h * p.q_hs;
    const bf16_t* Gh = (const bf16_t*)p.dout + (int64_t)h * p.do_hs;
    qs.load(Qh, p.q_ss, q0, lq);
    ds.load(Gh, p.do_ss, q0, lq);
    if (QTT) {
      qts.load(Qh, p.q_ss, q0, lq);
      dts.load(Gh, p.do_ss, q0, lq);
    }
  };
  int it = lq > 0 ? next_visible(0) : n_it;
  if (it < n_it) load(it);
  while (it < n_it) {
    const int h = g * p.group + it / n_qt;
    const int64_t q0 = (int64_t)(it % n_qt) * QT;
    __syncthreads();
    qs.store(sQ);
    ds.store(sdO);
    if (QTT) {
      qts.store(sQt);
      dts.store(sdOt);
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
    if (itn < n_it) load(itn);

    int64_t tq_lo, tq_hi;
    tile_bounds(it, tq_lo, tq_hi);
    const bool wave_skip = !wave_has_keys || (p.causal && tq_hi < wk_lo);
    if (!wave_skip) {
      const bool need_mask = (wkey0 + 32 > lk) || q0 + QT > lq || (p.causal && wk_hi > tq_lo);
      const TilePos tp(p.qm, q0, QT);
      // S and dP of both 32-query blocks are issued first; block 0's softmax
      // then runs on the vector ALU while block 1's MFMAs execute, and block 1's
      // softmax while block 0's dV/dK MFMAs execute
      f32x16 sacc[2], pacc[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        sacc[qb] = f32x16{};
        pacc[qb] = f32x16{};
        // operands of chunk c+1 are loaded while chunk c's MFMAs run
        bf16x8 aq[2], ao[2], bk[2], bv[2];
        auto ld = [&](int c, int slot) {
          const int off = (qb * 32 + srow) * QSTR + 16 * c + 8 * hi;
          aq[slot] = *(const bf16x8*)(sQ + off);
          ao[slot] = *(const bf16x8*)(sdO + off);
          bk[slot] = KVL ? *(const bf16x8*)(kop + 16 * c) : kreg[KVL ? 0 : c];
          bv[slot] = KVL ? *(const bf16x8*)(vop + 16 * c) : vreg[KVL ? 0 : c];
        };
        ld(0, 0);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          if (c + 1 < NC) ld(c + 1, (c + 1) & 1);
          sacc[qb] = mfma32(aq[c & 1], bk[c & 1], sacc[qb]);
          pacc[qb] = mfma32(ao[c & 1], bv[c & 1], pacc[qb]);
        }
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        // register r is query q0 + qb*32 + 16*(r/8) + 8*hi + r%8
        bf16x8 pP[2], pS[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int qo = qb * 32 + 16 * hf + 8 * hi;
          const f32x4 la = *(const f32x4*)(sL + qo), lb = *(const f32x4*)(sL + qo + 4);
          const f32x4 da = *(const f32x4*)(sDl + qo), db_ = *(const f32x4*)(sDl + qo + 4);
          bf16x8 p8, s8;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int r = 8 * hf + e;
            const float l2 = e < 4 ? la[e] : lb[e - 4];
            const float dl = e < 4 ? da[e] : db_[e - 4];
            float pr = __builtin_amdgcn_exp2f(fmaf(sacc[qb][r], p.scale_log2, -l2));
            if (need_mask) {
              const bool vis = (qo + e < tp.nvalid) & (tp.pos(qo + e) >= kmin);
              pr = vis ? pr : 0.f;
            }
            p8[e] = (bf16_t)pr;
            s8[e] = (bf16_t)(pr * (pacc[qb][r] - dl));
          }
          pP[hf] = p8;
          pS[hf] = s8;
        }
        // (db, hf) step i+1's transposed operands load while step i's MFMAs run
        bf16x8 ao[2], aq[2];
        auto ld = [&](int i, int slot) {
          const int db = i >> 1, cc = 2 * qb + (i & 1);
          ao[slot] = rows_operand<QTT, QSTR, QTSTR>(sdO, sdOt, 16 * cc, 32 * db, lane);
          aq[slot] = rows_operand<QTT, QSTR, QTSTR>(sQ, sQt, 16 * cc, 32 * db, lane);
        };
        ld(0, 0);
#pragma unroll
        for (int i = 0; i < 2 * ND; ++i) {
          if (i + 1 < 2 * ND) ld(i + 1, (i + 1) & 1);
          const int db = i >> 1, hf = i & 1;
          dvacc[db] = mfma32(ao[i & 1], pP[hf], dvacc[db]);
          dkacc[db] = mfma32(aq[i & 1], pS[hf], dkacc[db]);
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

int gcd_int(int a, int b) {
  while (b) {
    int t = a % b;
    a = b;
    b = t;
  }
  return a;
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
  if (p.qm.len > 0 && p.km.len > 0) {
    const int hpw = gcd_int(p.group, 4);
    const int rows_per_wg = (8 / hpw) * 32;
    const int n_qt = (int)((p.qm.len + rows_per_wg - 1) / rows_per_wg);
    const int64_t grid = (int64_t)p.hkv * (p.group / hpw) * n_qt;
    hipLaunchKernelGGL((bwd_dq_kernel<D>), dim3((unsigned)grid), dim3(512), 0, s, p, hpw, n_qt,
                       rows_per_wg);
  }
  const int n_kt = (int)((p.km.len + 127) / 128);
  const int64_t grid = (int64_t)p.hkv * n_kt;
  if (grid > 0)
    hipLaunchKernelGGL((bwd_dkv_kernel<D, (bool)RA_BWD_QTT, (bool)RA_BWD_KVL>), dim3((unsigned)grid),
                       dim3(256), 0, s, p, n_kt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_step_bwd(const StepParams& p, int dtype, int head_dim, hipStream_t s) {
  if (dtype == RA_BF16) return head_dim == 128 ? launch_mfma<128>(p, s) : launch_mfma<64>(p, s);
  return head_dim == 128 ? launch_simple<128, float>(p, s) : launch_simple<64, float>(p, s);
}
