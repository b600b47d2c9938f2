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
#include <string.h>

#include <type_traits>

#include "ra_internal.h"
#include "ra_tile.h"

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// the VALU kernels run the fp32 workload only
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
//     MULTI: every chunk of ch in turn (K, V and key map per chunk), dQ summed
//     in registers over the chunks and written (not accumulated) at the end.
template <int D, bool MULTI>
__device__ __forceinline__ void bwd_dq_body(const StepParams& p, int hpw, int n_qt,
                                            int rows_per_wg, const ChunkSet* ch) {
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
  const int64_t lq = p.qm.len;
  SegMap km = MULTI ? ch->km[0] : p.km;  // key map of the chunk being processed
  int64_t lk = km.len;
  const int64_t wg_r0 = (int64_t)qt * rows_per_wg;
  const int64_t row0 = wg_r0 + (int64_t)(wave / hpw) * 32;

  int64_t wq_lo = 0, wq_hi = -1, gq_lo, gq_hi;
  const bool wave_active = row0 < lq;
  if (wave_active) seg_bounds(p.qm, row0, row0 + 32 < lq ? row0 + 32 : lq, wq_lo, wq_hi);
  seg_bounds(p.qm, wg_r0, wg_r0 + rows_per_wg < lq ? wg_r0 + rows_per_wg : lq, gq_lo, gq_hi);

  const bf16_t* K = (const bf16_t*)(MULTI ? ch->k[0] : p.k) + (int64_t)g * p.k_hs;
  const bf16_t* V = (const bf16_t*)(MULTI ? ch->v[0] : p.v) + (int64_t)g * p.v_hs;

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

  KeyTiles<KT> kt_wg(km, p.causal, gq_lo, gq_hi);
  KeyTiles<KT> kt_w(km, p.causal, wq_lo, wq_hi);
  int n_kt = kt_wg.n;

  DmaSwz<KT, D, NW, 1> kst, vst;
  kst.init(p.k_ss, wave, lane);
  vst.init(p.v_ss, wave, lane);
  auto stage = [&](int t, auto b) {
    constexpr int B = decltype(b)::value;
    kst.issue(K, t * KT, (int)lk, B ? sK1 : sK0);
    vst.issue(V, t * KT, (int)lk, B ? sV1 : sV0);
  };

  // per-lane byte offsets in a swizzled tile: 16-byte row reads of chunk
  // 2*c + hi of row kb*32 + sigma(l32) (XOR 32 c), and transposing reads of
  // rows 16*cc + 8*hi + (gi / 4) (+4) at d = 32*db + 16*(grp & 1) + 4*(gi & 3)
  // (XOR 64 db)
  const int roff = swz_off<D>(srow, hi);
  const int grp = lane >> 4, gi = lane & 15;
  const int toff0 = swz_off<D>(8 * hi + (gi >> 2), 2 * (grp & 1) + ((gi & 3) >> 1)) + 8 * (gi & 1);
  const int toff1 = swz_off<D>(8 * hi + (gi >> 2) + 4, 2 * (grp & 1) + ((gi & 3) >> 1)) + 8 * (gi & 1);

  auto compute = [&](int t, auto b) {
    constexpr int B = decltype(b)::value;
    if (!wave_active) return;
    const char* cK = (const char*)(B ? sK1 : sK0);
    const char* cV = (const char*)(B ? sV1 : sV0);
    // S^T = K Q^T and dP^T = V dO^T; register r of key block kb is key
    // t*KT + kb*32 + 16*(r/8) + 8*hi + r%8
    f32x16 sacc[2] = {f32x16{}, f32x16{}}, pacc[2] = {f32x16{}, f32x16{}};
    // product i of 4 NC: step c = i / 4, key block kb = (i / 2) % 2, K (S) or
    // V (dP) for i % 2; each A operand is read AH products ahead of its use, in
    // a fixed issue order (each fence keeps the compiler from moving
    // instructions across it), so the LDS latency hides behind the products
    constexpr int NSD = 4 * NC, AH = 3;
    auto sd_op = [&](int i) -> bf16x8 {
      const int o = ((i / 2) % 2) * 32 * 2 * D + (roff ^ (32 * (i / 4)));
      return *(const bf16x8*)(((i & 1) ? cV : cK) + o);
    };
    bf16x8 ar[AH + 1];
#pragma unroll
    for (int i = 0; i < AH; ++i) ar[i] = sd_op(i);
#pragma unroll
    for (int i = 0; i < NSD; ++i) {
      if (i + AH < NSD) ar[(i + AH) % (AH + 1)] = sd_op(i + AH < NSD ? i + AH : 0);
      const int c = i / 4, kb = (i / 2) % 2;
      if (i & 1)
        pacc[kb] = mfma32(ar[i % (AH + 1)], doreg[c], pacc[kb]);
      else
        sacc[kb] = mfma32(ar[i % (AH + 1)], qreg[c], sacc[kb]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (!kt_w.mask_free(t)) {  // wave-uniform: one branch around branch-free code
      const TileRows tk(km, (int64_t)t * KT, KT);
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
    // 32*db + l32, read transposed, AH products ahead; product j of 4 ND is
    // cc = j / ND, db = j % ND, so consecutive MFMAs use different accumulators
    constexpr int NQ = 4 * ND;
    auto kt_op = [&](int j) -> bf16x8 {
      const char* a = cK + 16 * (j / ND) * 2 * D;
      const int dblk = 64 * (j % ND);  // byte XOR of the 32-wide d block
      return __builtin_shufflevector(ds_read_tr((const bf16_t*)(a + (toff0 ^ dblk))),
                                     ds_read_tr((const bf16_t*)(a + (toff1 ^ dblk))), 0, 1, 2,
                                     3, 4, 5, 6, 7);
    };
#pragma unroll
    for (int j = 0; j < AH; ++j) ar[j] = kt_op(j);
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      if (j + AH < NQ) ar[(j + AH) % (AH + 1)] = kt_op(j + AH < NQ ? j + AH : 0);
      const int cc = j / ND, db = j % ND;
      qacc[db] = mfma32(ar[j % (AH + 1)], dsk[cc >> 1][cc & 1], qacc[db]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  __syncthreads();  // zero-fill done before any DMA lands
  const int n_chunks = MULTI ? ch->n : 1;
  for (int c = 0; c < n_chunks; ++c) {
    if (MULTI && c > 0) {
      km = ch->km[c];
      lk = km.len;
      K = (const bf16_t*)ch->k[c] + (int64_t)g * p.k_hs;
      V = (const bf16_t*)ch->v[c] + (int64_t)g * p.v_hs;
      kt_wg = KeyTiles<KT>(km, p.causal, gq_lo, gq_hi);
      kt_w = KeyTiles<KT>(km, p.causal, wq_lo, wq_hi);
      n_kt = kt_wg.n;
      wait_vmem();
      __syncthreads();  // every wave is done with the previous chunk's buffers
    }
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
  }

  if (!qok) return;
  float* dq = p.o + qrow * p.o_ss + (int64_t)h * p.o_hs;
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4* ptr = (f32x4*)(dq + 32 * db + 8 * i + 4 * hi);
      f32x4 v4 = MULTI ? f32x4{} : *ptr;
#pragma unroll
      for (int j = 0; j < 4; ++j) v4[j] += qacc[db][4 * i + j] * p.scale;
      *ptr = v4;
    }
}

template <int D>
__global__ __launch_bounds__(512, 1) void bwd_dq_kernel(StepParams p, int hpw, int n_qt,
                                                        int rows_per_wg) {
  bwd_dq_body<D, false>(p, hpw, n_qt, rows_per_wg, nullptr);
}

template <int D>
__global__ __launch_bounds__(512, 1) void bwd_dq_chunks_kernel(StepParams p, int hpw, int n_qt,
                                                               int rows_per_wg, ChunkSet ch) {
  bwd_dq_body<D, true>(p, hpw, n_qt, rows_per_wg, &ch);
}

// (2) dK, dV, key-stationary, symmetric wave pairs: a workgroup of 8 waves
//      (two per SIMD) owns 128 keys of one KV head and walks the 64-row query
//      tiles of every query head of the group. Waves w and w ^ 4 share 32 keys;
//      wave half hf = w / 4 computes, for tile rows 32 hf .. 32 hf + 31,
//      S = Q K^T and dP = dO V^T (K and V of its key held as MFMA B operands),
//      then P = exp(S - LSE) and dS = P (dP - D) in fp32, each rounded once to
//      bf16, and hands them to its partner through LDS. After a barrier each
//      wave accumulates dV^T += dO^T P and dK^T += Q^T dS over all 64 rows for
//      the d columns 64 hf / (D/128) .. of its half, its own rows' P/dS from
//      registers and its partner's from LDS. Q and dO tiles reach LDS by DMA
//      one step ahead (two buffers each, XOR-swizzled), with the tile's LSE
//      (log2 units) and -D. Every dK/dV element has one writer.
//      The workgroup's KV head g and key block kt come from its caller.
template <int D>
__device__ __forceinline__ void bwd_dkv_body(const StepParams& p, const int g, const int kt) {
  constexpr int NW = 8;
  constexpr int KB = 128;      // keys per workgroup
  constexpr int QT = 64;       // query rows per tile
  constexpr int NC = D / 16;   // 16-wide d chunks (contraction steps of S and dP)
  constexpr int NDH = D / 64;  // 32-wide d blocks in a wave's half of d
  constexpr int TB = QT * D;   // elements per Q / dO tile
  constexpr int XB = 4 * 64 * 8;  // exchange elements per wave: 4 chunks x 64 lanes x 8
  // one LDS block at fixed byte offsets: the Q and dO tiles of buffers 0 and 1
  // in the low 64 KiB (so every read of a tile reaches its buffer through the
  // instruction's immediate offset, with no per-step address arithmetic), then
  // the P / dS hand-off, LSE * log2(e) (+inf: no contribution) and -D
  constexpr int TBB = TB * 2, XBB = NW * XB * 2;
  constexpr int oQ0 = 0, oG0 = TBB, oQ1 = 2 * TBB, oG1 = 3 * TBB, oX = 4 * TBB;
  constexpr int oL = oX + XBB, oD = oL + 2 * QT * 4, kLdsBytes = oD + 2 * QT * 4;
  static_assert(4 * TBB <= 65536, "tile buffers must lie within the immediate offset's reach");
  __shared__ __attribute__((aligned(1024))) char lds[kLdsBytes];
  bf16_t* const sQ0 = (bf16_t*)(lds + oQ0);
  bf16_t* const sQ1 = (bf16_t*)(lds + oQ1);
  bf16_t* const sG0 = (bf16_t*)(lds + oG0);
  bf16_t* const sG1 = (bf16_t*)(lds + oG1);
  bf16_t* const sX = (bf16_t*)(lds + oX);
  float(*const sL)[QT] = (float(*)[QT])(lds + oL);
  float(*const sD)[QT] = (float(*)[QT])(lds + oD);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int kw = wave & 3;     // key group of the pair
  const int hf = wave >> 2;    // row half (S, dP, P, dS) and d half (dK, dV)
  const int l32 = lane & 31, hi = lane >> 5;
  const int srow = sigma32(l32);

  const int64_t lq = p.qm.len, lk = p.km.len;
  const int64_t key0 = (int64_t)kt * KB;
  const int64_t key1 = key0 + KB < lk ? key0 + KB : lk;
  const int64_t wkey0 = key0 + kw * 32;
  const int64_t mykey = wkey0 + l32;
  const bool key_ok = mykey < lk;
  const int kpos = key_ok ? (int)seg_pos(p.km, mykey) : INT_MAX;
  int64_t gk_lo, gk_hi;
  seg_bounds(p.km, key0, key1, gk_lo, gk_hi);
  const bool wave_has_keys = wkey0 < lk;

  // K and V of this lane's key as B operands: d = 16c + 8*hi .. +8
  bf16x8 kreg[NC], vreg[NC];
  {
    const bf16_t* Kp = (const bf16_t*)p.k + (int64_t)g * p.k_hs + mykey * p.k_ss + 8 * hi;
    const bf16_t* Vp = (const bf16_t*)p.v + (int64_t)g * p.v_hs + mykey * p.v_ss + 8 * hi;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      bf16x8 z = {};
      kreg[c] = key_ok ? *(const bf16x8*)(Kp + 16 * c) : z;
      vreg[c] = key_ok ? *(const bf16x8*)(Vp + 16 * c) : z;
    }
  }
  // dV^T, dK^T of this lane's key: register r of block db is d row
  // (D/2) hf + 32 db + 8 (r/4) + 4 hi + r%4
  f32x16 dvacc[NDH], dkacc[NDH];
#pragma unroll
  for (int db = 0; db < NDH; ++db) {
    dvacc[db] = f32x16{};
    dkacc[db] = f32x16{};
  }

  // (query tile, query head) iterations: tiles in descending order with the
  // group's heads innermost (the workgroups of a KV head then read the same
  // Q / dO tiles at about the same time); hh == group marks the end
  const QueryTiles<QT> qt_wg(p.qm, p.causal, gk_lo, gk_hi);
  auto advance = [&](int& hh, int& t) {
    if (++hh < p.group) return;
    t = qt_wg.prev(t - 1);
    hh = t >= 0 ? 0 : p.group;
  };

  // waves 0-3 stage the Q tile, waves 4-7 the dO tile: each wave builds one
  // buffer descriptor per step (the address arithmetic is scalar, and all
  // eight waves issue it right after the step's barrier)
  const bool stages_q = wave < NW / 2;
  DmaSwz<QT, D, NW / 2, 3> dst;
  dst.init(stages_q ? p.q_ss : p.do_ss, wave & (NW / 2 - 1), lane);
  const bf16_t* const st_base = stages_q
                                    ? (const bf16_t*)p.q + (int64_t)g * p.group * p.q_hs
                                    : (const bf16_t*)p.dout + (int64_t)g * p.group * p.do_hs;
  const int64_t st_hs = stages_q ? p.q_hs : p.do_hs;
  auto stage = [&](int hh, int t, auto b) {
    constexpr int B = decltype(b)::value;
    bf16_t* const to = stages_q ? (B ? sQ1 : sQ0) : (B ? sG1 : sG0);
    dst.issue(st_base + hh * st_hs, t * QT, (int)lq, to);
  };
  // LSE and D of a tile: wave 0 loads them into registers one step before
  // they are written to LDS (at the start of the step before their tile's), so
  // the global loads never stall a step
  float pl = -INFINITY, pd = 0.f;
  auto load_ld = [&](int hh, int t) {
    if (wave == 0) {
      const int h = g * p.group + hh;
      const int64_t row = (int64_t)t * QT + lane;
      pl = -INFINITY;
      pd = 0.f;
      if (row < lq) {
        pl = p.lse_in[(int64_t)h * lq + row];
        pd = p.delta[(int64_t)h * lq + row];
      }
    }
  };
  auto store_ld = [&](auto b) {
    constexpr int B = decltype(b)::value;
    if (wave == 0) {
      sL[B][lane] = pl == -INFINITY ? INFINITY : pl * kLog2e;  // empty row: no contribution
      sD[B][lane] = -pd;
    }
  };

  // per-lane byte offsets in a swizzled tile: 16-byte row reads of chunk
  // 2c + hi of row 32 hf + sigma(l32) (XOR 32 c), and transposing reads of
  // rows 16 cq + 8 hi + gi/4 (+4) at d = 32 db + 16 (grp & 1) + 4 (gi & 3)
  // (XOR 64 db)
  const int grp = lane >> 4, gi = lane & 15;
  const int roff = 32 * hf * 2 * D + swz_off<D>(srow, hi);
  const int toff0 = swz_off<D>(8 * hi + (gi >> 2), 2 * (grp & 1) + ((gi & 3) >> 1)) + 8 * (gi & 1);
  const int toff1 = swz_off<D>(8 * hi + (gi >> 2) + 4, 2 * (grp & 1) + ((gi & 3) >> 1)) + 8 * (gi & 1);
  // the transposing reads' offsets for rows 32 hf' .. of the tile (hf' = hf:
  // this wave's rows, hf ^ 1: its partner's) and the wave's d block db (XOR 64
  // of the 32-wide block's index)
  int tro[2][NDH][2];
#pragma unroll
  for (int w = 0; w < 2; ++w)
#pragma unroll
    for (int db = 0; db < NDH; ++db) {
      const int rowb = 32 * (hf ^ w) * 2 * D, dblk = 64 * (NDH * hf + db);
      tro[w][db][0] = rowb + (toff0 ^ dblk);
      tro[w][db][1] = rowb + (toff1 ^ dblk);
    }
  // hand-off slots: chunk cq (16 rows) of wave w at sX[w][cq][lane][8]
  bf16_t* const x_mine = sX + wave * XB + lane * 8;
  const bf16_t* const x_partner = sX + (wave ^ 4) * XB + lane * 8;

  f32x16 sacc, pacc;
  bf16x8 pk[2], dsk[2];  // this wave's rows: chunks 2 hf + cc

  // phase 1 of a step: S, dP of this wave's rows; P, dS; hand-off
  auto phase1 = [&](int t, auto b) {
    constexpr int B = decltype(b)::value;
    const char* cQ = (const char*)(B ? sQ1 : sQ0);
    const char* cG = (const char*)(B ? sG1 : sG0);
    sacc = f32x16{};
    // dP accumulates onto -D of its rows (read first, ahead of the operands),
    // so the products leave dP - D: register r is row 32 hf + 16 (r/8) + 8 hi + r%8
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 nd = *(const f32x4*)(&sD[B][32 * hf + 16 * (j >> 1) + 8 * hi + 4 * (j & 1)]);
#pragma unroll
      for (int e = 0; e < 4; ++e) pacc[4 * j + e] = nd[e];
    }
    // the Q and dO row operands are read AH steps before their use, in a
    // fixed issue order (each fence keeps the compiler from moving
    // instructions across it), so the LDS latency hides behind the products
    constexpr int AH = 3;
    bf16x8 qa[AH + 1], ga[AH + 1];
    // LSE of row chunk cc: chunk 0's are read among the last products (after
    // the last operand read), chunk 1's at the start of chunk 0's vector work,
    // so neither waits on the LDS before its first use
    f32x4 ld[2][2];
    auto read_ld = [&](int cc) {
      const int qo = 32 * hf + 16 * cc + 8 * hi;
      ld[cc][0] = *(const f32x4*)(&sL[B][qo]);
      ld[cc][1] = *(const f32x4*)(&sL[B][qo + 4]);
    };
#pragma unroll
    for (int i = 0; i < AH; ++i) {
      qa[i] = *(const bf16x8*)(cQ + (roff ^ (32 * i)));
      ga[i] = *(const bf16x8*)(cG + (roff ^ (32 * i)));
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (c + AH < NC) {
        const int cn = c + AH < NC ? c + AH : 0;
        qa[cn % (AH + 1)] = *(const bf16x8*)(cQ + (roff ^ (32 * cn)));
        ga[cn % (AH + 1)] = *(const bf16x8*)(cG + (roff ^ (32 * cn)));
      }
      if (c == NC - AH) read_ld(0);
      sacc = mfma32(qa[c % (AH + 1)], kreg[c], sacc);
      pacc = mfma32(ga[c % (AH + 1)], vreg[c], pacc);
      __builtin_amdgcn_sched_barrier(0);
    }
    // register r is row 32 hf + 16 (r/8) + 8 hi + r%8 of the tile, the lane's key
    if (!qt_wg.mask_free(t)) {  // workgroup-uniform: one branch around branch-free selects
      const TileRows tq(p.qm, (int64_t)t * QT, QT);
      const QMaskBounds mb(tq, kpos, key_ok, 32 * hf + 8 * hi, p.causal);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool vis = mb.row_visible(16 * (r >> 3) + (r & 7));
        sacc[r] = vis ? sacc[r] : -INFINITY;
      }
    }
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      if (cc == 0) read_ld(1);
      float pv[8], sv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float l2 = e < 4 ? ld[cc][0][e] : ld[cc][1][e - 4];
        pv[e] = __builtin_amdgcn_exp2f(fmaf(sacc[8 * cc + e], p.scale_log2, -l2));
        sv[e] = pv[e] * pacc[8 * cc + e];  // P (dP - D)
      }
      pk[cc] = pack_bf16x8(pv);
      dsk[cc] = pack_bf16x8(sv);
      *(bf16x8*)(x_mine + (2 * cc) * 512) = pk[cc];
      *(bf16x8*)(x_mine + (2 * cc + 1) * 512) = dsk[cc];
    }
  };
  // phase 2: dV^T += dO^T P and dK^T += Q^T dS over the tile's 64 rows, for
  // this wave's d half; chunk cq of rows is this wave's (registers) when
  // cq / 2 == hf, else its partner's (LDS). Product m (of 8 NDH) is row chunk
  // k = m / (2 NDH) (this wave's chunks first), d block db = (m / 2) % NDH and
  // kind m % 2 (0: dV, 1: dK). Its A operand (dO^T or Q^T, read transposed)
  // is read AHEAD products before its use, in a fixed issue order, so the LDS
  // latency hides behind the products in flight.
  auto phase2 = [&](auto b) {
    constexpr int B = decltype(b)::value;
    const char* cQ = (const char*)(B ? sQ1 : sQ0);
    const char* cG = (const char*)(B ? sG1 : sG0);
    constexpr int NM = 8 * NDH;
    constexpr int AHEAD = 3;
    auto a_op = [&](int m) -> bf16x8 {
      const int k = m / (2 * NDH), db = (m / 2) % NDH;
      const char* a = ((m & 1) ? cQ : cG) + 16 * (k & 1) * 2 * D;
      return __builtin_shufflevector(ds_read_tr((const bf16_t*)(a + tro[k >> 1][db][0])),
                                     ds_read_tr((const bf16_t*)(a + tro[k >> 1][db][1])), 0, 1, 2,
                                     3, 4, 5, 6, 7);
    };
    bf16x8 ar[AHEAD + 1];
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) ar[i] = a_op(i);
    bf16x8 pb = pk[0], sb = dsk[0];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int k = m / (2 * NDH), db = (m / 2) % NDH;
      if (m + AHEAD < NM) ar[(m + AHEAD) % (AHEAD + 1)] = a_op(m + AHEAD < NM ? m + AHEAD : 0);
      if (m % (2 * NDH) == 0) {  // first product of a row chunk: its B operands
        const int cc = k & 1;
        pb = k < 2 ? pk[cc] : *(const bf16x8*)(x_partner + (2 * cc) * 512);
        sb = k < 2 ? dsk[cc] : *(const bf16x8*)(x_partner + (2 * cc + 1) * 512);
      }
      if ((m & 1) == 0)
        dvacc[db] = mfma32(ar[m % (AHEAD + 1)], pb, dvacc[db]);
      else
        dkacc[db] = mfma32(ar[m % (AHEAD + 1)], sb, dkacc[db]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Step i: tile i is in buffer i % 2 (landed at this step's first barrier);
  // the DMA of tile i + 1 goes to the other buffer (last read in the previous
  // step's phase 2, before this barrier).
  int ch = qt_wg.prev(qt_wg.n - 1) >= 0 ? 0 : p.group, ct = qt_wg.prev(qt_wg.n - 1);
  auto step = [&](auto b) {
    constexpr int B = decltype(b)::value;
    using NB = std::integral_constant<int, B ^ 1>;
    wait_vmem();
    __syncthreads();  // tile i, LSE/D of tile i visible; the other buffers free
    int nh = ch, nt = ct;
    advance(nh, nt);
    if (nh < p.group) {
      store_ld(NB{});  // tile i + 1's, loaded one step ago
      stage(nh, nt, NB{});
      int n2h = nh, n2t = nt;
      advance(n2h, n2t);
      if (n2h < p.group) load_ld(n2h, n2t);
    }
    if (wave_has_keys) phase1(ct, b);
    barrier_lds();  // the hand-off is visible
    if (wave_has_keys) phase2(b);
    ch = nh;
    ct = nt;
    return ch < p.group;
  };
  if (ch < p.group) {
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    stage(ch, ct, B0{});
    load_ld(ch, ct);
    wait_vmem();
    store_ld(B0{});
    {
      int nh = ch, nt = ct;
      advance(nh, nt);
      if (nh < p.group) load_ld(nh, nt);
    }
    // buffers alternate; unrolled so each buffer is a distinct array
    while (step(B0{}) && step(B1{})) {
    }
  }

  // ---- epilogue: lanes = keys, registers = d rows
  if (!key_ok) return;
  const int64_t obase = mykey * p.dk_ss + (int64_t)g * p.dk_hs + (D / 2) * hf;
#pragma unroll
  for (int db = 0; db < NDH; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4 a, c;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a[j] = dvacc[db][4 * i + j];
        c[j] = dkacc[db][4 * i + j] * p.scale;
      }
      f32x4* pv = (f32x4*)(p.dv + obase + 32 * db + 8 * i + 4 * hi);
      f32x4* pk4 = (f32x4*)(p.dk + obase + 32 * db + 8 * i + 4 * hi);
      if (p.dkv_accumulate) {
        a += *pv;
        c += *pk4;
      }
      *pv = a;
      *pk4 = c;
    }
}

// one ring step: workgroups in KV-head-major order, spread so that each XCD
// runs the key blocks of as few KV heads as possible (they share Q / dO)
template <int D>
__global__ __launch_bounds__(512, 1) void bwd_dkv_kernel(StepParams p, int n_kt) {
  const int logical = xcd_remap(blockIdx.x, p.hkv * n_kt, p.hkv);
  bwd_dkv_body<D>(p, logical / n_kt, logical % n_kt);
}

// The dK/dV outputs of every chunk of a ChunkSet, for one launch over all of
// them; kt0[c] is the first key block of chunk c in a KV head's sequence of
// blocks (kt0[n] = blocks per KV head).
struct DkvChunks {
  int32_t n;
  int32_t kt0[kMaxChunks + 1];
  float* dk[kMaxChunks];
  float* dv[kMaxChunks];
  int32_t acc[kMaxChunks];
};

// all chunks: per KV head, the key blocks of chunk 0, then chunk 1, ...; the
// same XCD spread as one step's launch, over the longer sequence
template <int D>
__global__ __launch_bounds__(512, 1) void bwd_dkv_chunks_kernel(StepParams p, ChunkSet ch,
                                                                DkvChunks dc) {
  const int per_g = dc.kt0[dc.n];
  const int logical = xcd_remap(blockIdx.x, p.hkv * per_g, p.hkv);
  const int g = logical / per_g;
  const int r = logical % per_g;
  int c = 0;
  while (c + 1 < dc.n && r >= dc.kt0[c + 1]) ++c;
  StepParams pc = p;
  pc.k = ch.k[c];
  pc.v = ch.v[c];
  pc.km = ch.km[c];
  pc.dk = dc.dk[c];
  pc.dv = dc.dv[c];
  pc.dkv_accumulate = dc.acc[c];
  bwd_dkv_body<D>(pc, g, r - dc.kt0[c]);
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

template <int D>
hipError_t launch_chunks(const StepParams& p, const ChunkSet& ch, float* const* dk,
                         float* const* dv, const int32_t* acc, hipStream_t s) {
  if (p.qm.len > 0) {
    const int hpw = gcd_int(p.group, 4);
    const int rows_per_wg = (8 / hpw) * 32;
    const int n_qt = (int)((p.qm.len + rows_per_wg - 1) / rows_per_wg);
    const int64_t grid = (int64_t)p.hkv * (p.group / hpw) * n_qt;
    hipLaunchKernelGGL((bwd_dq_chunks_kernel<D>), dim3((unsigned)grid), dim3(512), 0, s, p, hpw,
                       n_qt, rows_per_wg, ch);
  }
  static_assert(sizeof(StepParams) + sizeof(ChunkSet) + sizeof(DkvChunks) <= 4096,
                "kernel arguments above 4 KiB");
  DkvChunks dc;
  memset(&dc, 0, sizeof(dc));
  dc.n = ch.n;
  int64_t per_g = 0;
  for (int c = 0; c < ch.n; ++c) {
    dc.kt0[c] = (int32_t)per_g;
    per_g += (ch.km[c].len + 127) / 128;
    dc.dk[c] = dk[c];
    dc.dv[c] = dv[c];
    dc.acc[c] = acc[c];
  }
  dc.kt0[ch.n] = (int32_t)per_g;
  const int64_t grid = (int64_t)p.hkv * per_g;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  if (grid > 0)
    hipLaunchKernelGGL((bwd_dkv_chunks_kernel<D>), dim3((unsigned)grid), dim3(512), 0, s, p, ch,
                       dc);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_chunks(const StepParams& p, const ChunkSet& ch, float* const* dk,
                             float* const* dv, const int32_t* dkv_accumulate, int head_dim,
                             hipStream_t s) {
  return head_dim == 128 ? launch_chunks<128>(p, ch, dk, dv, dkv_accumulate, s)
                         : launch_chunks<64>(p, ch, dk, dv, dkv_accumulate, s);
}

hipError_t launch_step_bwd(const StepParams& p, int dtype, int head_dim, hipStream_t s) {
  if (dtype == RA_BF16) return head_dim == 128 ? launch_mfma<128>(p, s) : launch_mfma<64>(p, s);
  return head_dim == 128 ? launch_simple<128, float>(p, s) : launch_simple<64, float>(p, s);
}
