// Forward of one ring step: attention of the local query rows against one KV
// chunk, returning the unnormalised-free partial output O_step and its
// log-sum-exp (the per-step computation of ring attention, "Guide to
// LoongTrain", "The Communication Overhead and Causal Imbalance of Ring
// Attention"; scale 1/sqrt(d) and softmax(QK^T scale) V as in its "Step 3").
//
// bf16 path (gfx950 MFMA): a workgroup of 8 waves (two per SIMD) shares one KV
// head. Each wave owns 32 query rows of one query head; the waves of a
// workgroup are the grouped query heads that read the same K/V (GQA packing)
// and/or consecutive row blocks. K/V tiles of 64 keys are copied global -> LDS
// by DMA. Each wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 so that
// a lane owns one query column: the online softmax row max/sum are in-lane plus
// one exchange with the other half-wave (v_permlane32_swap). K rows are fed in
// the sigma order (ra_tile.h), so each 8-register chunk of exp2(S^T - m) covers
// 8 consecutive keys and, rounded to bf16, is directly the B operand of
// O^T += V^T P^T, whose A operand is read transposed from row-major V.
// Tiles whose keys are all later than the workgroup's queries are skipped;
// fully visible tiles run a mask-free copy of the tile code. The exponent shift
// (running max) moves only when a row's tile max exceeds it by 2^8, so O is
// rarely rescaled; the result is the same softmax, since LSE and the
// normalisation use the same shift.
//
// fp32 path: a plain VALU kernel (one or two lanes per query row), used for the
// fp32 workload and kept deliberately simple.
#include <limits.h>
#include <math.h>

#include <type_traits>

#include "ra_internal.h"
#include "ra_tile.h"

namespace {

constexpr float kLn2 = 0.69314718055994531f;

// the VALU kernels run the fp32 workload only
__device__ inline float to_f(float x) { return x; }

// Fold a step's row (O_s, L_s) into the running (O_a, L_a), as the merge of
// partial results over disjoint key sets does: m = max(La, Ls);
// L = m + ln(e^(La-m) + e^(Ls-m)), O = ca Oa + cs Os with ca = e^(La-L),
// cs = e^(Ls-L). A step row with no visible key (Ls = -inf) leaves the row as
// it is, so `update` is false and nothing is read or written for it.
struct MergeCoeffs {
  bool update;
  float ca, cs, lse;
};
__device__ inline MergeCoeffs merge_coeffs(float la, float ls) {
  MergeCoeffs r;
  r.update = ls != -INFINITY;
  const float m = fmaxf(la, ls);
  const float ea = r.update ? expf(la - m) : 1.f, es = r.update ? expf(ls - m) : 0.f;
  const float tot = ea + es, inv = 1.0f / tot;
  r.ca = ea * inv;
  r.cs = es * inv;
  r.lse = r.update ? m + logf(tot) : la;
  return r;
}

// ============================================================= VALU kernel
// TPR lanes per query row (D/64), each holding 64 of the d components.
template <int D, typename T, bool MERGE>
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
  const float ls = l > 0.f ? m + logf(l) : -INFINITY;
  float* orow = p.o + row * p.o_ss + h * p.o_hs + sub * 64;
  float* lrow = p.lse_out + (int64_t)h * p.qm.len + row;
  if (MERGE) {
    // both lanes of the row read L_a before one of them writes it back
    const MergeCoeffs mc = merge_coeffs(*lrow, ls);
    if (mc.update) {
#pragma unroll
      for (int x = 0; x < 64; ++x) orow[x] = mc.ca * orow[x] + mc.cs * (o[x] * inv);
      if (sub == 0) *lrow = mc.lse;
    }
    return;
  }
#pragma unroll
  for (int x = 0; x < 64; ++x) orow[x] = o[x] * inv;
  if (sub == 0) *lrow = ls;
}

// ============================================================= MFMA kernel
// A workgroup is 8 waves (two per SIMD); wave w owns 32 query rows of one query
// head. K and V tiles of 64 keys reach LDS by DMA, two buffers each (one
// barrier per tile). The loop is software-pipelined: while the softmax and
// O^T += V^T P^T of tile t run, the 16 MFMAs of S^T for the next tile are
// issued in the same basic block, in a fixed order that interleaves them with
// the O^T products and spreads the softmax between them, so vector and matrix
// work overlap inside each wave. Tiles use the XOR-swizzled row layout: K rows
// are read with 16-byte loads and V^T operands with ds_read_b64_tr_b16, both
// free of bank conflicts. Diagonal tiles and ragged tails add one branch-free
// masking block.

// Issue order of a forward step with NS score products: four score products,
// then O^T and score products alternating, then the remaining O^T products.
// Returns the product at position pos: score product i (< NS) or NS + O^T product j.
template <int NS>
__host__ __device__ constexpr int prod_at(int pos) {
  if (pos < 4) return pos;
  const int k = pos - 4;
  if (k < 2 * (NS - 4)) return (k % 2) ? 4 + k / 2 : NS + k / 2;
  return NS + (NS - 4) + (k - 2 * (NS - 4));
}
template <int NS>
__host__ __device__ constexpr int pos_of_o(int j) {
  return j < NS - 4 ? 4 + 2 * j : 4 + 2 * (NS - 4) + (j - (NS - 4));
}
// position after which softmax element e (chunk e / 8 of 8 keys) is computed:
// chunk k is spread over the positions before the first O^T product using it
template <int NS, int ND>
__host__ __device__ constexpr int elem_slot(int e) {
  const int k = e / 8;
  const int start = k == 0 ? 0 : pos_of_o<NS>((k - 1) * ND);
  const int n = pos_of_o<NS>(k * ND) - start;
  return start + ((e % 8) * n) / 8;
}
// two floats rounded to bf16 (round to nearest even) in one 32-bit register
__device__ __forceinline__ uint32_t pk2_bf16(float a, float b) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

// The body of the step kernels. MULTI: the whole ring in one launch, chunk c
// of ch in turn (K, V and key map per chunk), the running max, sum and output
// carried in registers from one chunk to the next and written once at the end.
template <int D, bool MERGE, bool MULTI>
__device__ __forceinline__ void fwd_mfma_body(const StepParams& p, int hpw, int n_qt,
                                              int rows_per_wg, const ChunkSet* ch) {
  constexpr int NW = 8;            // waves per workgroup
  constexpr int KT = 64;           // keys per LDS tile
  constexpr int TB = KT * D;       // elements per K / V tile (XOR-swizzled rows, no padding)
  constexpr int NC = D / 16;       // 16-wide d chunks (QK^T contraction steps)
  constexpr int ND = D / 32;       // 32-wide d blocks of O^T
  // log2-domain headroom before the running max is moved: P stays <= 2^8
  constexpr float kThresh = 8.f;
  __shared__ __attribute__((aligned(1024))) bf16_t sK0[TB];
  __shared__ __attribute__((aligned(1024))) bf16_t sK1[TB];
  __shared__ __attribute__((aligned(1024))) bf16_t sV0[TB];
  __shared__ __attribute__((aligned(1024))) bf16_t sV1[TB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int l32 = lane & 31, hi = lane >> 5;
  const int srow = sigma32(l32);

  // ---- workgroup -> (KV head, head subgroup, query tile); tiles of one KV head
  // share an XCD (and its L2); later (heavier) query tiles start first.
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

  // stale LDS must hold finite values: keys past the end are never read into
  // P != 0, but 0 * NaN would poison O
  for (int i = tid; i < TB / 8; i += NW * 64) {
    ((bf16x8*)sK0)[i] = bf16x8{};
    ((bf16x8*)sK1)[i] = bf16x8{};
    ((bf16x8*)sV0)[i] = bf16x8{};
    ((bf16x8*)sV1)[i] = bf16x8{};
  }

  // Q^T as the B operand: lane holds query column l32, d = 16c + 8*hi .. +8
  bf16x8 qreg[NC];
  const int64_t qrow = row0 + l32;
  const bool qok = qrow < lq;
  const int qpos = qok ? (int)seg_pos(p.qm, qrow) : -1;
  const int qlim = (p.causal || !qok) ? qpos : INT_MAX;  // last visible key position
  {
    const bf16_t* Q = (const bf16_t*)p.q + qrow * p.q_ss + (int64_t)h * p.q_hs + 8 * hi;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      bf16x8 z = {};
      qreg[c] = qok ? *(const bf16x8*)(Q + 16 * c) : z;
    }
  }

  f32x16 oacc[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY;  // running max (log2 units) used as the exponent shift
  float l_run = 0.f;        // running sum of this half-wave's keys

  // visible key tiles of the workgroup, and the tiles this wave must mask
  KeyTiles<KT> kt_wg(km, p.causal, gq_lo, gq_hi);
  KeyTiles<KT> kt_w(km, p.causal, wq_lo, wq_hi);
  int n_kt = kt_wg.n;
  auto next_visible = [&](int t) { return kt_wg.next(t); };

  DmaSwz<KT, D, NW, MERGE ? 5 : 0> kst, vst;
  kst.init(p.k_ss, wave, lane);
  vst.init(p.v_ss, wave, lane);
  auto kbuf = [&](auto b) -> bf16_t* {
    constexpr int B = decltype(b)::value;
    return B == 0 ? sK0 : sK1;
  };
  auto vbuf = [&](auto b) -> bf16_t* {
    constexpr int B = decltype(b)::value;
    return B == 0 ? sV0 : sV1;
  };
  auto stage_k = [&](int t, auto b) { kst.issue(K, t * KT, (int)lk, kbuf(b)); };
  auto stage_v = [&](int t, auto b) { vst.issue(V, t * KT, (int)lk, vbuf(b)); };

  // per-lane LDS offsets (elements); everything else is an immediate offset
  // per-lane byte offsets in a swizzled tile: 16-byte reads of chunk 2*c + hi
  // of row kb*32 + sigma(l32) (K), and transposing reads of rows
  // 16*cc + 8*hi + (gi / 4) (+4) at d = 32*db + 16*(grp & 1) + 4*(gi & 3) (V)
  const int roff = swz_off<D>(srow, hi);
  const int grp = lane >> 4, gi = lane & 15;
  const int toff0 = swz_off<D>(8 * hi + (gi >> 2), 2 * (grp & 1) + ((gi & 3) >> 1)) + 8 * (gi & 1);
  const int toff1 = swz_off<D>(8 * hi + (gi >> 2) + 4, 2 * (grp & 1) + ((gi & 3) >> 1)) + 8 * (gi & 1);

  // S^T = K Q^T of the tile in buffer b; register r of key block kb is key
  // t*KT + kb*32 + 16*(r/8) + 8*hi + r%8
  auto scores = [&](auto b, f32x16 (&sacc)[2]) {
    const char* cK = (const char*)kbuf(b);
    sacc[0] = f32x16{};
    sacc[1] = f32x16{};
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        sacc[kb] = mfma32(*(const bf16x8*)(cK + kb * 32 * 2 * D + (roff ^ (32 * c))), qreg[c], sacc[kb]);
  };
  // mask scores of tile t for this wave's queries (keys past the end, and
  // causally later keys) and move the exponent shift if the tile needs it
  // max of 16 raw scores of a lane (a tree of depth 3)
  auto max16 = [](const f32x16& v) {
    const float a = fmax3(v[0], v[1], v[2]), b = fmax3(v[3], v[4], v[5]);
    const float c = fmax3(v[6], v[7], v[8]), d = fmax3(v[9], v[10], v[11]);
    const float e = fmax3(v[12], v[13], v[14]);
    return __builtin_fmaxf(fmax3(a, b, c), fmax3(d, e, v[15]));
  };
  // mx_pre (have_pre): the lane's max of the tile's unmasked scores, computed
  // in the step's block; tiles that need a mask recompute it after masking
  auto prepare = [&](int t, f32x16 (&sacc)[2], float mx_pre, bool have_pre) {
    const bool need_mask = !wave_active || !kt_w.mask_free(t);
    if (need_mask) {  // wave-uniform: one branch around branch-free code
      // the lane part (8*hi) of each key offset is folded into the per-tile
      // bounds so each register compares against a constant
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
    // tile row max on raw scores (scale > 0), over both lane halves
    float mx = (have_pre && !need_mask) ? mx_pre : __builtin_fmaxf(max16(sacc[0]), max16(sacc[1]));
    mx = max_halves(mx);
    const float mt = mx * p.scale_log2;
    // the shift moves only when a row's max outgrows it by kThresh (rarely after
    // the first tiles); P = exp2(s - m_run) <= 2^kThresh otherwise
    if (__any(mt > m_run + kThresh)) {
      const float m_new = __builtin_fmaxf(m_run, mt);
      const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < ND; ++db) oacc[db] *= alpha;
    }
  };
  // One step's products in a fixed issue order: the 2*NC score products of the
  // next tile (A = K row chunk, one 16-byte read) and the 4*ND O^T products of
  // this tile (A = V^T, two transposing reads) alternate after four score
  // products; each A operand is read AH products ahead of its use, and the
  // softmax of this tile (32 scores per lane in four chunks of 8 keys) is spread
  // over the products before the first O^T product that needs each chunk.
  // Fences keep the compiler from moving instructions across products, and the
  // empty asm statements keep each softmax piece where it is placed (the
  // instruction selector would otherwise sink it to its first use). Without the
  // fixed order, the compiler read the V^T operands of two of the three unrolled
  // steps right before their products and waited for each read.
  constexpr int NS = 2 * NC, NO = 4 * ND, NPR = NS + NO, AH = 3;
  auto block = [&](auto bc, auto bn, const f32x16 (&sacc)[2], f32x16 (&snew)[2], float& mxo) {
    const char* cK = (const char*)kbuf(bn);
    const char* cV = (const char*)vbuf(bc);
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    snew[0] = f32x16{};
    snew[1] = f32x16{};
    auto opnd = [&](int pos) -> bf16x8 {
      const int pr = prod_at<NS>(pos);
      if (pr < NS) return *(const bf16x8*)(cK + (pr % 2) * 32 * 2 * D + (roff ^ (32 * (pr / 2))));
      const int j = pr - NS;
      const char* a = cV + 16 * (j / ND) * 2 * D;
      const int dblk = 64 * (j % ND);
      return __builtin_shufflevector(ds_read_tr((const bf16_t*)(a + (toff0 ^ dblk))),
                                     ds_read_tr((const bf16_t*)(a + (toff1 ^ dblk))), 0, 1, 2, 3,
                                     4, 5, 6, 7);
    };
    float pe[32], mx0 = 0.f;
    uint32_t pw[16];
    bf16x8 pkc[4];
    float rs0 = 0.f, rs1 = 0.f;
    bf16x8 ar[AH + 1];
#pragma unroll
    for (int i = 0; i < AH; ++i) ar[i] = opnd(i);
#pragma unroll
    for (int pos = 0; pos < NPR; ++pos) {
      if (pos + AH < NPR) ar[(pos + AH) % (AH + 1)] = opnd(pos + AH < NPR ? pos + AH : 0);
      const int pr = prod_at<NS>(pos);
      if (pr < NS) {
        snew[pr % 2] = mfma32(ar[pos % (AH + 1)], qreg[pr / 2], snew[pr % 2]);
      } else {
        const int j = pr - NS;
        oacc[j % ND] = mfma32(ar[pos % (AH + 1)], pkc[j / ND], oacc[j % ND]);
      }
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        if (elem_slot<NS, ND>(e) != pos) continue;
        pe[e] = __builtin_amdgcn_exp2f(fmaf(sacc[e / 16][e % 16], p.scale_log2, -m_use));
        if (e & 1) {
          rs1 += pe[e];
          pw[e / 2] = pk2_bf16(pe[e - 1], pe[e]);
          asm volatile("" : "+v"(pw[e / 2]), "+v"(rs1));
        } else {
          rs0 += pe[e];
          asm volatile("" : "+v"(rs0));
        }
        if (e % 8 == 7)
          pkc[e / 8] = __builtin_bit_cast(
              bf16x8, u32x4{pw[e / 2 - 3], pw[e / 2 - 2], pw[e / 2 - 1], pw[e / 2]});
      }
      // the lane's max of the new (unmasked) scores, among the last O^T products,
      // once the score products have completed: off the path to the next step
      if (pos == NPR - 3) {
        mx0 = max16(snew[0]);
        asm volatile("" : "+v"(mx0));
      }
      if (pos == NPR - 2) {
        mxo = __builtin_fmaxf(mx0, max16(snew[1]));
        asm volatile("" : "+v"(mxo));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run += rs0 + rs1;
  };

  // One pipeline step. On entry sc holds the prepared scores of tile t, whose V
  // is in buffer bv, and the K of the next tile tn is in bk. K and V rotate
  // through two buffers each: after the barrier (which makes the previous
  // step's loads visible and ends all reads of that step) the K of the tile
  // after tn goes into bkl (tile t's K buffer) and the V of tn into bvl (the
  // V buffer read one step ago). Scores of tn are computed (unconditionally:
  // past the end they are discarded) in the same block as tile t's softmax and
  // O update; the loop is unrolled so each buffer is a distinct array (the
  // compiler then knows a load into one does not alias reads of another).
  f32x16 sc[2], sn[2];
  int t = next_visible(0), tn = n_kt;
  auto step = [&](auto bv, auto bk, auto bkl, auto bvl) {
    wait_vmem();
    __syncthreads();
    const int tn2 = tn < n_kt ? next_visible(tn + 1) : n_kt;
    if (tn2 < n_kt) stage_k(tn2, bkl);
    if (tn < n_kt) stage_v(tn, bvl);
    float mxn = 0.f;
    block(bv, bk, sc, sn, mxn);
    t = tn;
    tn = tn2;
    if (t < n_kt) {
      sc[0] = sn[0];
      sc[1] = sn[1];
      prepare(t, sc, mxn, true);
    }
    return t < n_kt;
  };

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
      t = next_visible(0);
      tn = n_kt;
      __syncthreads();  // every wave is done with the previous chunk's buffers
    }
    if (t < n_kt) {
      using B0 = std::integral_constant<int, 0>;
      using B1 = std::integral_constant<int, 1>;
      stage_k(t, B0{});
      stage_v(t, B0{});
      tn = next_visible(t + 1);
      if (tn < n_kt) stage_k(tn, B1{});
      wait_vmem();
      __syncthreads();
      scores(B0{}, sc);
      prepare(t, sc, 0.f, false);
      while (step(B0{}, B1{}, B0{}, B1{}) && step(B1{}, B0{}, B1{}, B0{})) {
      }
    }
  }

  // ---- epilogue: normalise, write O_step [row][h][d] and LSE_step [h][row],
  // or fold them into O_acc and LSE_acc
  if (!wave_active) return;
  const float ltot = sum_halves(l_run);
  if (qok) {
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    const float ls = ltot > 0.f ? (m_run + log2f(ltot)) * kLn2 : -INFINITY;
    float* orow = p.o + qrow * p.o_ss + (int64_t)h * p.o_hs;
    float* lrow = p.lse_out + (int64_t)h * lq + qrow;
    if (MERGE) {
      // both lane halves read L_a before one of them writes it back
      const MergeCoeffs mc = merge_coeffs(*lrow, ls);
      if (mc.update) {
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            f32x4* pa = (f32x4*)(orow + 32 * db + 8 * i + 4 * hi);
            f32x4 a = *pa;
#pragma unroll
            for (int j = 0; j < 4; ++j) a[j] = mc.ca * a[j] + mc.cs * (oacc[db][4 * i + j] * inv);
            *pa = a;
          }
        if (hi == 0) *lrow = mc.lse;
      }
    } else {
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f32x4 v4;
#pragma unroll
          for (int j = 0; j < 4; ++j) v4[j] = oacc[db][4 * i + j] * inv;
          *(f32x4*)(orow + 32 * db + 8 * i + 4 * hi) = v4;
        }
      if (hi == 0) *lrow = ls;
    }
  }
}

template <int D, bool MERGE>
__global__ __launch_bounds__(512, 1) void fwd_mfma_kernel(StepParams p, int hpw, int n_qt,
                                                          int rows_per_wg) {
  fwd_mfma_body<D, MERGE, false>(p, hpw, n_qt, rows_per_wg, nullptr);
}

template <int D>
__global__ __launch_bounds__(512, 1) void fwd_chunks_kernel(StepParams p, int hpw, int n_qt,
                                                            int rows_per_wg, ChunkSet ch) {
  fwd_mfma_body<D, false, true>(p, hpw, n_qt, rows_per_wg, &ch);
}

int gcd_int(int a, int b) {
  while (b) {
    int t = a % b;
    a = b;
    b = t;
  }
  return a;
}

template <int D>
hipError_t launch_mfma(const StepParams& p, hipStream_t s) {
  const int hpw = gcd_int(p.group, 4);  // query heads per row block (GQA packing)
  const int rows_per_wg = (8 / hpw) * 32;
  const int n_qt = (int)((p.qm.len + rows_per_wg - 1) / rows_per_wg);
  const int64_t grid = (int64_t)p.hkv * (p.group / hpw) * n_qt;
  if (grid == 0) return hipSuccess;
  if (p.merge)
    hipLaunchKernelGGL((fwd_mfma_kernel<D, true>), dim3((unsigned)grid), dim3(512), 0, s, p, hpw,
                       n_qt, rows_per_wg);
  else
    hipLaunchKernelGGL((fwd_mfma_kernel<D, false>), dim3((unsigned)grid), dim3(512), 0, s, p, hpw,
                       n_qt, rows_per_wg);
  return hipGetLastError();
}

template <int D>
hipError_t launch_chunks(const StepParams& p, const ChunkSet& ch, hipStream_t s) {
  const int hpw = gcd_int(p.group, 4);
  const int rows_per_wg = (8 / hpw) * 32;
  const int n_qt = (int)((p.qm.len + rows_per_wg - 1) / rows_per_wg);
  const int64_t grid = (int64_t)p.hkv * (p.group / hpw) * n_qt;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((fwd_chunks_kernel<D>), dim3((unsigned)grid), dim3(512), 0, s, p, hpw, n_qt,
                     rows_per_wg, ch);
  return hipGetLastError();
}

template <int D, typename T>
hipError_t launch_simple(const StepParams& p, hipStream_t s) {
  constexpr int RPB = 64 / (D / 64);
  const unsigned gx = (unsigned)((p.qm.len + RPB - 1) / RPB);
  if (p.merge)
    hipLaunchKernelGGL((fwd_simple_kernel<D, T, true>), dim3(gx, p.hq), dim3(64), 0, s, p);
  else
    hipLaunchKernelGGL((fwd_simple_kernel<D, T, false>), dim3(gx, p.hq), dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_chunks(const StepParams& p, const ChunkSet& ch, int head_dim,
                             hipStream_t s) {
  return head_dim == 128 ? launch_chunks<128>(p, ch, s) : launch_chunks<64>(p, ch, s);
}

hipError_t launch_step_fwd(const StepParams& p, int dtype, int head_dim, hipStream_t s) {
  if (dtype == RA_BF16) {
    if (head_dim == 128) return launch_mfma<128>(p, s);
    return launch_mfma<64>(p, s);
  }
  if (head_dim == 128) return launch_simple<128, float>(p, s);
  return launch_simple<64, float>(p, s);
}
