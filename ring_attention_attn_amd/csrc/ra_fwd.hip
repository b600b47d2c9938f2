// Forward of one ring step: attention of the local query rows against one KV
// chunk, returning the unnormalised-free partial output O_step and its
// log-sum-exp (the per-step computation of ring attention, "Guide to
// LoongTrain", "The Communication Overhead and Causal Imbalance of Ring
// Attention"; scale 1/sqrt(d) and softmax(QK^T scale) V as in its "Step 3").
//
// bf16 path (gfx950 MFMA): a workgroup of 4 waves shares one KV head. Each wave
// owns 32*QB query rows of one query head; the waves of a workgroup are the
// grouped query heads that read the same K/V (GQA packing) and/or consecutive
// row blocks. K/V tiles of 64 keys are staged in LDS; each wave computes
// S^T = K Q^T with v_mfma_f32_32x32x16_bf16 so that a lane owns one query
// column: the row max/sum of the online softmax are in-lane plus one exchange
// with the other half-wave. exp2(S^T - m) is rounded to bf16 and used in place
// as the B operand of O^T += V^T P^T; V^T comes from LDS through the
// transposing read ds_read_b64_tr_b16. Tiles whose keys are all later than the
// workgroup's queries are skipped; fully visible tiles run without masking.
//
// fp32 path: a plain VALU kernel (one or two lanes per query row), used for the
// fp32 workload and kept deliberately simple.
#include <math.h>

#include "ra_internal.h"

namespace {

constexpr float kLn2 = 0.69314718055994531f;

__device__ inline float to_f(bf16_t x) { return (float)x; }
__device__ inline float to_f(float x) { return x; }

// ============================================================= VALU kernel
// TPR lanes per query row (D/64), each holding 64 of the d components.
template <int D, typename T>
__global__ __launch_bounds__(64) void fwd_simple_kernel(StepParams p) {
  constexpr int TPR = D / 64;
  constexpr int RPB = 64 / TPR;  // rows per block
  constexpr int KT = 32;
  __shared__ float sK[KT][D];
  __shared__ float sV[KT][D];
  const int h = blockIdx.y;
  const int g = h / p.group;
  const int sub = threadIdx.x % TPR;
  const int64_t r0 = (int64_t)blockIdx.x * RPB;
  const int64_t row = r0 + threadIdx.x / TPR;
  const bool valid = row < p.qm.len;
  const int64_t qpos = valid ? seg_pos(p.qm, row) : -1;
  int64_t qlo, qhi;
  seg_bounds(p.qm, r0, r0 + RPB < p.qm.len ? r0 + RPB : p.qm.len, qlo, qhi);
  const T* Q = (const T*)p.q;
  const T* K = (const T*)p.k;
  const T* V = (const T*)p.v;
  float q[64], o[64];
#pragma unroll
  for (int x = 0; x < 64; ++x) {
    q[x] = valid ? to_f(Q[row * p.q_ss + h * p.q_hs + sub * 64 + x]) : 0.f;
    o[x] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int64_t k0 = 0; k0 < p.km.len; k0 += KT) {
    const int64_t k1 = k0 + KT < p.km.len ? k0 + KT : p.km.len;
    int64_t klo, khi;
    seg_bounds(p.km, k0, k1, klo, khi);
    if (p.causal && klo > qhi) continue;  // uniform over the block
    __syncthreads();
    for (int i = threadIdx.x; i < KT * D; i += 64) {
      const int kr = i / D, x = i % D;
      const int64_t key = k0 + kr;
      sK[kr][x] = key < k1 ? to_f(K[key * p.k_ss + g * p.k_hs + x]) : 0.f;
      sV[kr][x] = key < k1 ? to_f(V[key * p.v_ss + g * p.v_hs + x]) : 0.f;
    }
    __syncthreads();
    for (int j = 0; j < (int)(k1 - k0); ++j) {
      const int64_t kpos = seg_pos(p.km, k0 + j);
      float s = 0.f;
#pragma unroll
      for (int x = 0; x < 64; ++x) s += q[x] * sK[j][sub * 64 + x];
      if (TPR == 2) s += __shfl_xor(s, 1);
      if (!valid || (p.causal && kpos > qpos)) continue;
      s *= p.scale;
      if (s > m) {
        const float c = expf(m - s);
        l *= c;
#pragma unroll
        for (int x = 0; x < 64; ++x) o[x] *= c;
        m = s;
      }
      const float e = expf(s - m);
      l += e;
#pragma unroll
      for (int x = 0; x < 64; ++x) o[x] += e * sV[j][sub * 64 + x];
    }
  }
  if (!valid) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int x = 0; x < 64; ++x) p.o[row * p.o_ss + h * p.o_hs + sub * 64 + x] = o[x] * inv;
  if (sub == 0) p.lse_out[(int64_t)h * p.qm.len + row] = l > 0.f ? m + logf(l) : -INFINITY;
}

// ============================================================= MFMA kernel
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ inline bf16x4 ds_read_tr(const bf16_t* lds_ptr) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_ptr));
  return __builtin_bit_cast(bf16x4, r);
}

template <int D, int QB>
__global__ __launch_bounds__(256, 1) void fwd_mfma_kernel(StepParams p, int hpw, int n_qt,
                                                          int rows_per_wg) {
  constexpr int KT = 64;         // keys per LDS tile
  constexpr int KSTR = D + 8;    // LDS row strides (elements), chosen against bank conflicts
  constexpr int VSTR = D + 16;
  constexpr int NC = D / 16;     // 16-wide d chunks (QK^T contraction steps)
  constexpr int ND = D / 32;     // 32-wide d blocks of O^T
  constexpr int CPR = D / 8;     // 16-byte chunks per K/V row
  constexpr int NLD = KT * CPR / 256;
  __shared__ __attribute__((aligned(16))) bf16_t sK[KT * KSTR];
  __shared__ __attribute__((aligned(16))) bf16_t sV[KT * VSTR];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;

  // ---- workgroup -> (KV head, head subgroup, query tile); same-KV-head tiles
  // are placed on the same XCD (workgroups go round-robin over the 8 XCDs).
  const int nsub = p.group / hpw;
  const int total = p.hkv * nsub * n_qt;
  const int w = blockIdx.x;
  const int logical = (total % 8 == 0) ? (w % 8) * (total / 8) + (w / 8) : w;
  const int gh = logical / n_qt;
  const int qt = n_qt - 1 - (logical % n_qt);  // later (heavier) rows first
  const int g = gh / nsub, hs = gh % nsub;
  const int h = g * p.group + hs * hpw + (wave % hpw);
  const int64_t lq = p.qm.len, lk = p.km.len;
  const int64_t wg_r0 = (int64_t)qt * rows_per_wg;
  const int64_t row0 = wg_r0 + (int64_t)(wave / hpw) * 32 * QB;

  int64_t wq_lo = 0, wq_hi = -1, gq_lo, gq_hi;
  const bool wave_active = row0 < lq;
  if (wave_active) seg_bounds(p.qm, row0, row0 + 32 * QB < lq ? row0 + 32 * QB : lq, wq_lo, wq_hi);
  seg_bounds(p.qm, wg_r0, wg_r0 + rows_per_wg < lq ? wg_r0 + rows_per_wg : lq, gq_lo, gq_hi);

  const bf16_t* Q = (const bf16_t*)p.q;
  const bf16_t* K = (const bf16_t*)p.k + (int64_t)g * p.k_hs;
  const bf16_t* V = (const bf16_t*)p.v + (int64_t)g * p.v_hs;

  // Q^T as the B operand: lane holds query column l32, d = 16c + 8*hi .. +8
  bf16x8 qreg[QB][NC];
  int qpos[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int64_t row = row0 + qb * 32 + l32;
    const bool ok = row < lq;
    qpos[qb] = ok ? (int)seg_pos(p.qm, row) : -1;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      bf16x8 z = {};
      qreg[qb][c] = ok ? *(const bf16x8*)(Q + row * p.q_ss + (int64_t)h * p.q_hs + 16 * c + 8 * hi) : z;
    }
  }

  f32x16 oacc[QB][ND];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < ND; ++db) oacc[qb][db] = f32x16{};
  }

  const int n_kt = (int)((lk + KT - 1) / KT);
  auto tile_bounds = [&](int t, int64_t& lo, int64_t& hi_) {
    const int64_t k0 = (int64_t)t * KT;
    seg_bounds(p.km, k0, k0 + KT < lk ? k0 + KT : lk, lo, hi_);
  };
  auto next_visible = [&](int t) {
    while (t < n_kt) {
      if (!p.causal) return t;
      int64_t lo, hh;
      tile_bounds(t, lo, hh);
      if (lo <= gq_hi) return t;
      ++t;
    }
    return t;
  };

  bf16x8 kr[NLD], vr[NLD];
  auto load_regs = [&](int t) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int c = i * 256 + tid;
      const int r = c / CPR, col = (c % CPR) * 8;
      const int64_t key = (int64_t)t * KT + r;
      bf16x8 z = {};
      kr[i] = key < lk ? *(const bf16x8*)(K + key * p.k_ss + col) : z;
      vr[i] = key < lk ? *(const bf16x8*)(V + key * p.v_ss + col) : z;
    }
  };
  auto store_lds = [&]() {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int c = i * 256 + tid;
      const int r = c / CPR, col = (c % CPR) * 8;
      *(bf16x8*)(sK + r * KSTR + col) = kr[i];
      *(bf16x8*)(sV + r * VSTR + col) = vr[i];
    }
  };

  // transposing-read lane roles (see ds_read_tr): 16-lane group grp, member i
  const int grp = lane >> 4, gi = lane & 15;
  const int tr_key = 4 * (grp >> 1) + (gi >> 2);  // + 16*chunk (+8 for the 2nd read)
  const int tr_d = 16 * (grp & 1) + 4 * (gi & 3);   // + 32*db

  int t = next_visible(0);
  if (t < n_kt) load_regs(t);
  while (t < n_kt) {
    __syncthreads();
    store_lds();
    __syncthreads();
    const int tn = next_visible(t + 1);
    if (tn < n_kt) load_regs(tn);

    int64_t klo, khi;
    tile_bounds(t, klo, khi);
    const bool wave_skip = !wave_active || (p.causal && klo > wq_hi);
    if (!wave_skip) {
      const bool ragged = (int64_t)(t + 1) * KT > lk;
      const bool need_mask = ragged || (p.causal && khi > wq_lo);
      // ---- S^T = K Q^T : two 32-key blocks x QB 32-query blocks
      f32x16 sacc[2][QB];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) sacc[kb][qb] = f32x16{};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 a = *(const bf16x8*)(sK + (kb * 32 + l32) * KSTR + 16 * c + 8 * hi);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            sacc[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[qb][c], sacc[kb][qb], 0, 0, 0);
        }
      }
      // ---- scale, mask, online softmax (exp2 domain)
      bf16x8 pk[2][QB][2];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float s = sacc[kb][qb][r] * p.scale_log2;
            if (need_mask) {
              const int64_t key = (int64_t)t * KT + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
              const bool vis = key < lk && (!p.causal || seg_pos(p.km, key) <= qpos[qb]);
              s = vis ? s : -INFINITY;
            }
            sacc[kb][qb][r] = s;
            mx = fmaxf(mx, s);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run[qb], mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_use);
        m_run[qb] = m_new;
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            bf16x8 v8;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float pe = __builtin_amdgcn_exp2f(sacc[kb][qb][hf * 8 + e] - m_use);
              rs += pe;
              v8[e] = (bf16_t)pe;
            }
            pk[kb][qb][hf] = v8;
          }
        l_run[qb] = l_run[qb] * alpha + rs;
#pragma unroll
        for (int db = 0; db < ND; ++db) oacc[qb][db] *= alpha;
      }
      // ---- O^T += V^T P^T : V^T (d x 16 keys) by transposing LDS reads
#pragma unroll
      for (int db = 0; db < ND; ++db) {
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const bf16_t* base = sV + (16 * cc + tr_key) * VSTR + 32 * db + tr_d;
          const bf16x4 lo4 = ds_read_tr(base);
          const bf16x4 hi4 = ds_read_tr(base + 8 * VSTR);
          const bf16x8 a = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[cc >> 1][qb][cc & 1],
                                                                   oacc[qb][db], 0, 0, 0);
        }
      }
    }
    t = tn;
  }

  // ---- epilogue: normalise, write O_step [row][h][d] and LSE_step [h][row]
  if (!wave_active) return;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float ltot = l_run[qb] + __shfl_xor(l_run[qb], 32);
    const int64_t row = row0 + qb * 32 + l32;
    if (row < lq) {
      const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
      float* orow = p.o + row * p.o_ss + (int64_t)h * p.o_hs;
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f32x4 v4;
#pragma unroll
          for (int j = 0; j < 4; ++j) v4[j] = oacc[qb][db][4 * i + j] * inv;
          *(f32x4*)(orow + 32 * db + 8 * i + 4 * hi) = v4;
        }
      if (hi == 0)
        p.lse_out[(int64_t)h * lq + row] = ltot > 0.f ? (m_run[qb] + log2f(ltot)) * kLn2 : -INFINITY;
    }
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

template <int D, int QB>
hipError_t launch_mfma(const StepParams& p, hipStream_t s) {
  const int hpw = gcd_int(p.group, 4);
  const int rb = 4 / hpw;
  const int rows_per_wg = rb * 32 * QB;
  const int n_qt = (int)((p.qm.len + rows_per_wg - 1) / rows_per_wg);
  const int64_t grid = (int64_t)p.hkv * (p.group / hpw) * n_qt;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((fwd_mfma_kernel<D, QB>), dim3((unsigned)grid), dim3(256), 0, s, p, hpw, n_qt,
                     rows_per_wg);
  return hipGetLastError();
}

template <int D, typename T>
hipError_t launch_simple(const StepParams& p, hipStream_t s) {
  constexpr int RPB = 64 / (D / 64);
  const unsigned gx = (unsigned)((p.qm.len + RPB - 1) / RPB);
  hipLaunchKernelGGL((fwd_simple_kernel<D, T>), dim3(gx, p.hq), dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_step_fwd(const StepParams& p, int dtype, int head_dim, hipStream_t s) {
  if (dtype == RA_BF16) {
    if (head_dim == 128) return launch_mfma<128, 1>(p, s);
    return launch_mfma<64, 1>(p, s);
  }
  if (head_dim == 128) return launch_simple<128, float>(p, s);
  return launch_simple<64, float>(p, s);
}
