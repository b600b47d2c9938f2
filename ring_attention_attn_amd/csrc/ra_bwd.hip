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
// (1) dQ, query-stationary: a workgroup of 8 waves (two per SIMD) shares each
//     64-key K/V tile (LDS-DMA, double-buffered, one barrier per tile); a wave
//     owns 32 query rows of one head. S^T = K Q^T and dP^T = V dO^T put a query
//     in each lane, so LSE and D are per-lane scalars; dS^T (bf16, 8
//     consecutive keys per register chunk thanks to the sigma row order) is the
//     B operand of dQ^T += K^T dS^T, whose A operand is read transposed from
//     the row-major K tile. Both tiles use the XOR-swizzled layout, so the
//     16-byte row reads and the transposing reads are free of bank conflicts.
//     dq_acc is read-modify-written once per row at the end: no atomics.
template <int D>
__global__ __launch_bounds__(512, 1) void bwd_dq_kernel(StepParams p, int hpw, int n_qt,
                                                        int rows_per_wg) {
  constexpr int NW = 8;
  constexpr int KT = 64;
  constexpr int TB = KT * D;     // elements per K / V tile
  constexpr int NC = D / 16;
  constexpr int ND = D / 32;
  __shared__ __attribute__((aligned(1024))) bf16_t sK0[TB];
  __shared__ __attribute__((aligned(1024))) bf16_t sK1[TB];
  __shared__ __attribute__((aligned(1024))) bf16_t sV0[TB];
  __shared__ __attribute__((aligned(1024))) bf16_t sV1[TB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int l32 = lane & 31, hi = lane >> 5;
  const int srow = sigma32(l32);

  const int nsub = p.group / hpw;
  const int total = p.hkv * nsub * n_qt;
  const int logical = xcd_remap(blockIdx.x, total, p.hkv * nsub);
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
  for (int i = tid; i < TB / 8; i += NW * 64) {
    ((bf16x8*)sK0)[i] = bf16x8{};
    ((bf16x8*)sK1)[i] = bf16x8{};
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

  DmaSwz<KT, D, NW, 1> kst, vst;
  kst.init(p.k_ss, wave, lane);
  vst.init(p.v_ss, wave, lane);
  auto stage = [&](int t, auto b) {
    constexpr int B = decltype(b)::value;
    kst.issue(K, p.k_ss, (int64_t)t * KT, lk, B ? sK1 : sK0);
    vst.issue(V, p.v_ss, (int64_t)t * KT, lk, B ? sV1 : sV0);
  };

  // per-lane byte offsets in a swizzled tile: 16-byte row reads of chunk
  // 2*c + hi of row kb*32 + sigma(l32), and transposing reads of rows
  // 16*cc + 8*hi + (gi / 4) (+4) at d = 32*db + 16*(grp & 1) + 4*(gi & 3)
  int roff[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) roff[c] = swz_off<D>(srow, 2 * c + hi);
  const int grp = lane >> 4, gi = lane & 15;
  int toff[2][ND];
#pragma unroll
  for (int sh = 0; sh < 2; ++sh)
#pragma unroll
    for (int db = 0; db < ND; ++db)
      toff[sh][db] = swz_off<D>(8 * hi + (gi >> 2) + 4 * sh, 4 * db + 2 * (grp & 1) + ((gi & 3) >> 1)) +
                     8 * (gi & 1);

  auto compute = [&](int t, auto b) {
    constexpr int B = decltype(b)::value;
    if (!wave_active) return;
    const char* cK = (const char*)(B ? sK1 : sK0);
    const char* cV = (const char*)(B ? sV1 : sV0);
    // S^T = K Q^T and dP^T = V dO^T; register r of key block kb is key
    // t*KT + kb*32 + 16*(r/8) + 8*hi + r%8
    f32x16 sacc[2] = {f32x16{}, f32x16{}}, pacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int o = kb * 32 * 2 * D + roff[c];
        sacc[kb] = mfma32(*(const bf16x8*)(cK + o), qreg[c], sacc[kb]);
        pacc[kb] = mfma32(*(const bf16x8*)(cV + o), doreg[c], pacc[kb]);
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
        const char* a = cK + 16 * cc * 2 * D;
        const bf16x4 lo4 = ds_read_tr((const bf16_t*)(a + toff[0][db]));
        const bf16x4 hi4 = ds_read_tr((const bf16_t*)(a + toff[1][db]));
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

// dK/dV kernel tuning: LDS reads issued ahead of the score products, and the
// wave priority of the P waves (whose chain sets the step time)
#ifndef RA_DKV_AHEAD
#define RA_DKV_AHEAD 8
#endif
#ifndef RA_DKV_PPRIO
#define RA_DKV_PPRIO 1
#endif

// (2) dK, dV, key-stationary: a workgroup of 8 waves (two per SIMD) owns 128
//     keys of one KV head and walks the 64-row query tiles of every query head
//     of the group. The waves come in pairs on the same 32 keys: the P wave
//     computes S = Q K^T (K held as the MFMA B operand), P = exp(S - LSE) and
//     dV^T += dO^T P, and hands P (bf16) to its partner through LDS; the
//     partner (V held) computes dP = dO V^T of the same tile in the same step
//     and, one step later, dS = P (dP - D) and dK^T += Q^T dS. Each wave keeps
//     one accumulator set (the dK wave also one tile of dP), so both roles fit
//     two waves per SIMD, and no product is computed twice. The dK wave
//     starts each step with the dS products of the previous tile, the P wave
//     with its score products, so their VALU-heavy phases do not coincide.
//     Q tiles reach LDS by DMA two steps ahead (four rotating buffers), dO
//     tiles one step ahead (two buffers), both XOR-swizzled, with the tile's
//     LSE (log2 units) and D; one barrier per step. Query rows are fed in
//     sigma order, so P and dS are directly B operands of the dV / dK
//     products, whose A operands are read transposed from the same tiles.
//     Each dK/dV element has one writer.
template <int D>
__global__ __launch_bounds__(512, 1) void bwd_dkv_kernel(StepParams p, int n_kt) {
  constexpr int NW = 8;
  constexpr int KB = 128;  // keys per workgroup
  constexpr int QT = 64;   // query rows per tile
  constexpr int NC = D / 16;
  constexpr int ND = D / 32;
  constexpr int TB = QT * D;  // elements per Q / dO tile
  constexpr int PB = QT * 32;  // elements of P per key group
  __shared__ __attribute__((aligned(1024))) bf16_t sQ0[TB];
  __shared__ __attribute__((aligned(1024))) bf16_t sQ1[TB];
  __shared__ __attribute__((aligned(1024))) bf16_t sQ2[TB];
  __shared__ __attribute__((aligned(1024))) bf16_t sQ3[TB];
  __shared__ __attribute__((aligned(1024))) bf16_t sG0[TB];
  __shared__ __attribute__((aligned(1024))) bf16_t sG1[TB];
  __shared__ __attribute__((aligned(1024))) bf16_t sP[2 * 4 * PB];  // two slots
  __shared__ __attribute__((aligned(16))) float sL[2][QT];  // LSE * log2(e) (+inf: no contribution)
  __shared__ __attribute__((aligned(16))) float sD[4][QT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const bool pwave = wave < 4;  // role: P / dV (else dS / dK)
  const int kw = wave & 3;      // key group of the wave pair
  const int l32 = lane & 31, hi = lane >> 5;
  const int srow = sigma32(l32);

  const int logical = xcd_remap(blockIdx.x, p.hkv * n_kt, p.hkv);
  const int g = logical / n_kt;
  const int kt = logical % n_kt;  // earlier keys (seen by more queries) first
  const int64_t lq = p.qm.len, lk = p.km.len;
  const int64_t key0 = (int64_t)kt * KB;
  const int64_t key1 = key0 + KB < lk ? key0 + KB : lk;
  const int64_t wkey0 = key0 + kw * 32;
  const int64_t mykey = wkey0 + l32;
  const bool key_ok = mykey < lk;
  const int kpos = key_ok ? (int)seg_pos(p.km, mykey) : INT_MAX;
  int64_t gk_lo, gk_hi, wk_lo = 0, wk_hi = 0;
  seg_bounds(p.km, key0, key1, gk_lo, gk_hi);
  const bool wave_has_keys = wkey0 < lk;
  if (wave_has_keys) seg_bounds(p.km, wkey0, wkey0 + 32 < lk ? wkey0 + 32 : lk, wk_lo, wk_hi);

  // K (P wave) or V (dK wave) of this lane's key as the B operand: d = 16c + 8*hi .. +8
  bf16x8 breg[NC];
  {
    const bf16_t* Bp = pwave ? (const bf16_t*)p.k + (int64_t)g * p.k_hs + mykey * p.k_ss
                             : (const bf16_t*)p.v + (int64_t)g * p.v_hs + mykey * p.v_ss;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      bf16x8 z = {};
      breg[c] = key_ok ? *(const bf16x8*)(Bp + 8 * hi + 16 * c) : z;
    }
  }
  f32x16 acc[ND];  // dV^T (P wave) or dK^T (dK wave): lane = key, registers = d
#pragma unroll
  for (int db = 0; db < ND; ++db) acc[db] = f32x16{};

  // iterations: (query tile t, query head of the group hh) pairs, tiles in
  // descending order with the heads innermost, so the workgroups of one KV
  // head read the same Q / dO tiles at about the same time until each reaches
  // its first visible tile (the visible tiles are suffixes, different for each
  // key block on the diagonal step; a shared order keeps them in L2);
  // hh == group marks the end
  const QueryTiles<QT> qt_wg(p.qm, p.causal, gk_lo, gk_hi);
  const QueryTiles<QT> qt_w(p.qm, p.causal, wk_lo, wk_hi);
  const int t_last = qt_wg.prev(qt_wg.n - 1);
  // the visible (tile, head) after (t, hh), or (-1, group)
  auto advance = [&](int& hh, int& t) {
    if (++hh < p.group) return;
    t = qt_wg.prev(t - 1);
    hh = t >= 0 ? 0 : p.group;
  };

  DmaSwz<QT, D, NW, 2> qst, gst;
  qst.init(p.q_ss, wave, lane);
  gst.init(p.do_ss, wave, lane);
  // buffers by step position (compile-time, so DMA into one buffer never
  // orders reads of another)
  auto qbuf = [&](auto b) -> bf16_t* {
    constexpr int B = decltype(b)::value & 3;
    return B == 0 ? sQ0 : (B == 1 ? sQ1 : (B == 2 ? sQ2 : sQ3));
  };
  auto gbuf = [&](auto b) -> bf16_t* {
    constexpr int B = decltype(b)::value & 1;
    return B == 0 ? sG0 : sG1;
  };
  // (an invalid tile is still issued, with no rows in range, so that every
  // step issues the same number of loads; it fills a free buffer with zeros)
  auto stage_q = [&](int hh, int t, auto b, bool valid) {
    const int h = g * p.group + (valid ? hh : 0);
    const int64_t q0 = valid ? (int64_t)t * QT : 0;
    qst.issue_untracked((const bf16_t*)p.q + (int64_t)h * p.q_hs, p.q_ss, q0, valid ? lq : q0,
                        qbuf(b));
  };
  auto stage_g = [&](int hh, int t, auto b) {
    const int h = g * p.group + hh;
    gst.issue_untracked((const bf16_t*)p.dout + (int64_t)h * p.do_hs, p.do_ss, (int64_t)t * QT, lq,
                        gbuf(b));
  };
  // LSE and D of a tile: wave 0 loads them into registers two steps before the
  // tile is used and writes them to LDS at the end of the next step, so the
  // loads never stall a step
  float pl = -INFINITY, pd = 0.f;  // loaded one step ago
  float nl = -INFINITY, nd = 0.f;  // loaded in this step
  auto load_ld = [&](int hh, int t, float& l, float& d) {
    if (wave == 0) {
      const int h = g * p.group + hh;
      const int64_t row = (int64_t)t * QT + lane;
      l = -INFINITY;
      d = 0.f;
      if (row < lq) {
        l = p.lse_in[(int64_t)h * lq + row];
        d = p.delta[(int64_t)h * lq + row];
      }
    }
  };
  auto store_ld = [&](auto b, float l, float d) {
    constexpr int B = decltype(b)::value;
    if (wave == 0) {
      sL[B & 1][lane] = l == -INFINITY ? INFINITY : l * kLog2e;  // empty row: no contribution
      sD[B & 3][lane] = d;
    }
  };

  // per-lane byte offsets in a swizzled tile: 16-byte row reads of chunk
  // 2*c + hi of row qb*32 + sigma(l32), and transposing reads of rows
  // 16*cq + 8*hi + (gi / 4) (+4) at d = 32*db + 16*(grp & 1) + 4*(gi & 3).
  // The swizzle is an XOR on the chunk index, so the offset for chunk c
  // (block db) is that of chunk 0 (block 0) XOR 32*c (64*db); the bases are
  // passed through an opaque copy every step, so the derived offsets are
  // formed where they are used instead of being held across the loop.
  const int grp = lane >> 4, gi = lane & 15;
  const int roff_base = swz_off<D>(srow, hi);
  const int toff_base0 = swz_off<D>(8 * hi + (gi >> 2), 2 * (grp & 1) + ((gi & 3) >> 1)) + 8 * (gi & 1);
  const int toff_base1 = swz_off<D>(8 * hi + (gi >> 2) + 4, 2 * (grp & 1) + ((gi & 3) >> 1)) + 8 * (gi & 1);
  int roff0 = roff_base, toff0 = toff_base0, toff1 = toff_base1;
  auto refresh_offsets = [&]() {
    roff0 = roff_base;
    toff0 = toff_base0;
    toff1 = toff_base1;
    asm volatile("" : "+v"(roff0), "+v"(toff0), "+v"(toff1));
  };
  // P hand-off slot of this lane: block (qb, hf) of key group kw, 16 bytes per lane
  const int p_lane = kw * PB + lane * 8;

  // A x (B operand) over the tile's two 32-row query blocks: register r of
  // block qb is query row qb*32 + 16*(r/8) + 8*hi + r%8, the lane's key
  auto row_products = [&](const char* tile, f32x16 (&x)[2]) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      x[qb] = f32x16{};
#pragma unroll
      for (int c = 0; c < NC; ++c)
        x[qb] = mfma32(*(const bf16x8*)(tile + qb * 32 * 2 * D + (roff0 ^ (32 * c))), breg[c], x[qb]);
    }
  };
  // acc^T += tile^T B' over 16 query rows cq (B' = P or dS chunk in bf16)
  auto col_products = [&](const char* tile, int cq, const bf16x8& bv) {
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      const char* a = tile + 16 * cq * 2 * D;
      const bf16x8 av = __builtin_shufflevector(ds_read_tr((const bf16_t*)(a + (toff0 ^ (64 * db)))),
                                                ds_read_tr((const bf16_t*)(a + (toff1 ^ (64 * db)))), 0,
                                                1, 2, 3, 4, 5, 6, 7);
      acc[db] = mfma32(av, bv, acc[db]);
    }
  };

  // score block: S = Q K^T of the tile in buffer b into sc, with the tile
  // reads issued AH products ahead
  f32x16 sc[2];
  auto scores = [&](auto b) {
    row_products((const char*)qbuf(b), sc);
    constexpr int AH = RA_DKV_AHEAD < 2 * NC ? RA_DKV_AHEAD : 2 * NC;
    if (AH > 0) {
      __builtin_amdgcn_sched_group_barrier(0x100, AH, 0);  // LDS reads
#pragma unroll
      for (int i = 0; i < 2 * NC - AH; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
      }
      __builtin_amdgcn_sched_group_barrier(0x008, AH, 0);
    }
  };
  // P wave at step position I (tile i): S, mask, P -> LDS slot I % 2,
  // dV^T += dO^T P
  auto p_step = [&](int t, auto pos) {
    constexpr int I = decltype(pos)::value;
    const char* cG = (const char*)gbuf(std::integral_constant<int, I>{});
    scores(std::integral_constant<int, I>{});
    // masking of the diagonal / ragged tiles: a uniform branch around
    // branch-free selects that rewrite the scores in place (a whole second copy
    // of the step would keep the accumulators in other registers and copy them
    // back at the join)
    if (!qt_w.mask_free(t)) {
      const TileRows tq(p.qm, (int64_t)t * QT, QT);
      const QMaskBounds mb(tq, kpos, key_ok, 8 * hi, p.causal);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const bool vis = mb.row_visible(qb * 32 + 16 * (r >> 3) + (r & 7));
          sc[qb][r] = vis ? sc[qb][r] : -INFINITY;
        }
    }
    bf16_t* sp = sP + (I & 1) * 4 * PB + p_lane;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int qo = qb * 32 + 16 * hf + 8 * hi;
        const f32x4 la = *(const f32x4*)(&sL[I & 1][qo]), lb = *(const f32x4*)(&sL[I & 1][qo + 4]);
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float l2 = e < 4 ? la[e] : lb[e - 4];
          pv[e] = __builtin_amdgcn_exp2f(fmaf(sc[qb][8 * hf + e], p.scale_log2, -l2));
        }
        const bf16x8 pk = pack_bf16x8(pv);
        *(bf16x8*)(sp + (2 * qb + hf) * 512) = pk;
        col_products(cG, 2 * qb + hf, pk);
      }
  };
  // dK wave at step position I: dS of tile i - 1 (its dP in dp, its P in
  // slot (I - 1) % 2), dK^T += Q^T dS, then dP of tile i into dp
  // (unconditionally: past the last tile it is discarded). The dS products
  // come first, so the pair's VALU-heavy phases (softmax here, dS there) fall
  // against the other wave's matrix products.
  f32x16 dp[2];
  auto k_step = [&](auto pos, auto ds_tag) {
    constexpr int I = decltype(pos)::value;
    constexpr bool DS = decltype(ds_tag)::value;
    if (DS) {
      const char* cQ = (const char*)qbuf(std::integral_constant<int, I + 3>{});
      const bf16_t* sp = sP + ((I + 1) & 1) * 4 * PB + p_lane;
      constexpr int DSL = (I + 3) & 3;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int qo = qb * 32 + 16 * hf + 8 * hi;
          const f32x4 da = *(const f32x4*)(&sD[DSL][qo]), db_ = *(const f32x4*)(&sD[DSL][qo + 4]);
          const bf16x8 pk = *(const bf16x8*)(sp + (2 * qb + hf) * 512);
          float sv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float dl = e < 4 ? da[e] : db_[e - 4];
            sv[e] = (float)pk[e] * (dp[qb][8 * hf + e] - dl);
          }
          col_products(cQ, 2 * qb + hf, pack_bf16x8(sv));
        }
    }
    row_products((const char*)gbuf(std::integral_constant<int, I>{}), dp);
  };

  // Step i (position I = i % 4): Q and dO of tile i have landed at this
  // step's barrier (Q of tile i + 1 may still be in flight); the DMA of dO of
  // tile i + 1 goes to the dO buffer read by both roles one step ago, then
  // that of Q of tile i + 2 to the Q buffer last read by the dK waves one step
  // ago. The two roles run
  // separate loops with the same barrier sequence, so each role's registers
  // are allocated on their own.
  int ch = t_last >= 0 ? 0 : p.group, ct = t_last;  // tile i
  int nh = ch, nt = ct;                                    // tile i + 1
  if (ch < p.group) advance(nh, nt);
  bool have_prev = false;
  // The Q DMA of the previous step is the last vector-memory operation issued
  // and is read no earlier than the next step: the waits leave it in flight.
  constexpr int QDMA = DmaSwz<QT, D, NW, 2>::PER;  // DMA instructions per lane per tile
  static_assert((QT * 2 * D / 1024) % NW == 0, "every wave issues QDMA loads per tile");
  auto step = [&](auto pos, auto role) {
    constexpr int I = decltype(pos)::value;
    constexpr bool PW = decltype(role)::value;
    wait_vmem_n<QDMA>();
    barrier_lds();  // Q(i), dO(i), LSE(i), D(i-1), P(i-1) visible; DMA targets free
    refresh_offsets();
    const bool cur = ch < p.group;
    const bool nxt = nh < p.group;
    int n2h = nh, n2t = nt;
    if (nxt) advance(n2h, n2t);
    if (nxt) stage_g(nh, nt, std::integral_constant<int, I + 1>{});
    if (n2h < p.group) load_ld(n2h, n2t, nl, nd);
    asm volatile("" ::: "memory");  // keep the Q DMA last
    stage_q(n2h, n2t, std::integral_constant<int, I + 2>{}, n2h < p.group);
    if (wave_has_keys) {
      if (PW) {
        if (cur) p_step(ct, pos);
      } else {
        if (have_prev)
          k_step(pos, std::true_type{});
        else
          k_step(pos, std::false_type{});
      }
    }
    if (nxt) store_ld(std::integral_constant<int, I + 1>{}, pl, pd);  // visible at the next barrier
    pl = nl;
    pd = nd;
    have_prev = cur;
    ch = nh;
    ct = nt;
    nh = n2h;
    nt = n2t;
    return have_prev;
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using P2 = std::integral_constant<int, 2>;
  using P3 = std::integral_constant<int, 3>;
  if (ch < p.group) {
    stage_q(ch, ct, P0{}, true);
    stage_q(nh, nt, P1{}, nh < p.group);
    stage_g(ch, ct, P0{});
    load_ld(ch, ct, pl, pd);
    store_ld(P0{}, pl, pd);
    if (nh < p.group) load_ld(nh, nt, pl, pd);
    wait_vmem();
    __syncthreads();
    // four-step unroll: buffer indices are compile-time constants
    if (pwave) {
      const std::true_type r{};
      if (RA_DKV_PPRIO) __builtin_amdgcn_s_setprio(RA_DKV_PPRIO);
      while (step(P0{}, r) && step(P1{}, r) && step(P2{}, r) && step(P3{}, r)) {
      }
    } else {
      const std::false_type r{};
      while (step(P0{}, r) && step(P1{}, r) && step(P2{}, r) && step(P3{}, r)) {
      }
    }
    wait_vmem();  // the last (empty) Q DMA lands before the workgroup's LDS is released
  }

  // ---- epilogue: lanes = keys, registers = d rows 8*(r/4) + 4*hi + r%4
  if (!key_ok) return;
  float* dst = (pwave ? p.dv : p.dk) + mykey * p.dk_ss + (int64_t)g * p.dk_hs;
  const float out_scale = pwave ? 1.f : p.scale;
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4 a;
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] = acc[db][4 * i + j] * out_scale;
      f32x4* pa = (f32x4*)(dst + 32 * db + 8 * i + 4 * hi);
      if (p.dkv_accumulate) a += *pa;
      *pa = a;
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
    hipLaunchKernelGGL((bwd_dkv_kernel<D>), dim3((unsigned)grid), dim3(512), 0, s, p, n_kt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_step_bwd(const StepParams& p, int dtype, int head_dim, hipStream_t s) {
  if (dtype == RA_BF16) return head_dim == 128 ? launch_mfma<128>(p, s) : launch_mfma<64>(p, s);
  return head_dim == 128 ? launch_simple<128, float>(p, s) : launch_simple<64, float>(p, s);
}
