// C ABI entry points of libringattn: host-side validation, index maps and
// dispatch to the kernel launchers. Nothing here allocates device memory.
#include <math.h>
#include <string.h>

#include "ra_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(int dtype) { return dtype == RA_BF16 ? 2 : 4; }

// strides of a [rows][heads][d] tensor: last dim contiguous, rows 16-byte aligned,
// and no two (row, head) vectors overlap when there is more than one.
ra_status check_strides(int64_t ss, int64_t hs, int64_t rows, int32_t heads, int32_t d, int eb) {
  if (ss < 0 || hs < 0) return RA_EINVAL;
  if (heads > 1 && hs < d) return RA_EINVAL;
  if (rows > 1 && ss < d) return RA_EINVAL;
  // one of the two nestings: [rows][heads][d] (ss >= hs * heads) or [heads][rows][d]
  // (hs >= ss * rows), padding allowed; written as divisions so no product overflows
  if (rows > 1 && heads > 1 && ss / heads < hs && hs / rows < ss) return RA_EINVAL;
  int64_t per16 = 16 / eb;
  if ((ss % per16) != 0 || (hs % per16) != 0) return RA_EALIGN;
  // the kernels address a tile of up to 64 rows from its first row with 32-bit
  // byte offsets (buffer loads), so 64 row strides must stay below 2^31 bytes
  if (ss > ((int64_t)1 << 31) / (64 * eb) - 2 * d) return RA_EUNSUPPORTED;
  return RA_OK;
}

ra_status check_seg(int32_t nseg, int64_t seg_len, const int64_t* pos) {
  if (nseg != 1 && nseg != 2) return RA_EINVAL;
  if (seg_len < 0) return RA_EINVAL;
  for (int i = 0; i < nseg; ++i) {
    if (pos[i] < 0 || pos[i] > (INT64_MAX / 4)) return RA_EINVAL;
    if (pos[i] + seg_len > (int64_t)INT32_MAX - 64) return RA_EUNSUPPORTED;  // kernels use int32
  }
  return RA_OK;
}

SegMap make_map(int32_t nseg, int64_t seg_len, const int64_t* pos) {
  SegMap m;
  m.pos0 = pos[0];
  m.pos1 = nseg == 2 ? pos[1] : pos[0] + seg_len;
  m.seg_len = seg_len;
  m.len = (int64_t)nseg * seg_len;
  return m;
}

ra_status from_hip(hipError_t e) { return e == hipSuccess ? RA_OK : RA_EDEVICE; }

}  // namespace

extern "C" {

const char* ra_status_str(ra_status s) {
  switch (s) {
    case RA_OK: return "RA_OK";
    case RA_EINVAL: return "RA_EINVAL: invalid argument";
    case RA_EUNSUPPORTED: return "RA_EUNSUPPORTED: unsupported configuration";
    case RA_EALIGN: return "RA_EALIGN: pointer or stride not 16-byte aligned";
    case RA_EDEVICE: return "RA_EDEVICE: kernel launch failed";
  }
  return "unknown ra_status";
}

ra_status ra_validate_step(const ra_step_desc* d, int32_t for_bwd) {
  if (!d) return RA_EINVAL;
  if (d->dtype != RA_BF16 && d->dtype != RA_F32) return RA_EINVAL;
  if (d->head_dim != 64 && d->head_dim != 128) return RA_EUNSUPPORTED;
  if (d->hq < 1 || d->hkv < 1 || d->hq % d->hkv != 0) return RA_EINVAL;
  if (d->causal != 0 && d->causal != 1) return RA_EINVAL;
  if (!isfinite(d->scale) || !(d->scale > 0.f)) return RA_EINVAL;
  if (d->dkv_accumulate != 0 && d->dkv_accumulate != 1) return RA_EINVAL;
  ra_status st;
  if ((st = check_seg(d->q_nseg, d->q_seg_len, d->q_seg_pos)) != RA_OK) return st;
  if ((st = check_seg(d->k_nseg, d->k_seg_len, d->k_seg_pos)) != RA_OK) return st;
  const int64_t lq = (int64_t)d->q_nseg * d->q_seg_len;
  const int64_t lk = (int64_t)d->k_nseg * d->k_seg_len;
  // row counts, tile offsets and positions are int32 in the kernels
  if (lq > INT32_MAX - 256 || lk > INT32_MAX - 256) return RA_EUNSUPPORTED;
  const int eb = elem_bytes(d->dtype);
  const int D = d->head_dim;
  if ((st = check_strides(d->q_ss, d->q_hs, lq, d->hq, D, eb)) != RA_OK) return st;
  if ((st = check_strides(d->k_ss, d->k_hs, lk, d->hkv, D, eb)) != RA_OK) return st;
  if ((st = check_strides(d->v_ss, d->v_hs, lk, d->hkv, D, eb)) != RA_OK) return st;
  if ((st = check_strides(d->o_ss, d->o_hs, lq, d->hq, D, 4)) != RA_OK) return st;
  if (for_bwd) {
    if ((st = check_strides(d->do_ss, d->do_hs, lq, d->hq, D, eb)) != RA_OK) return st;
    if ((st = check_strides(d->dk_ss, d->dk_hs, lk, d->hkv, D, 4)) != RA_OK) return st;
  }
  return RA_OK;
}

static StepParams make_params(const ra_step_desc* d) {
  StepParams p;
  memset(&p, 0, sizeof(p));
  p.q_ss = d->q_ss; p.q_hs = d->q_hs;
  p.k_ss = d->k_ss; p.k_hs = d->k_hs;
  p.v_ss = d->v_ss; p.v_hs = d->v_hs;
  p.o_ss = d->o_ss; p.o_hs = d->o_hs;
  p.do_ss = d->do_ss; p.do_hs = d->do_hs;
  p.dk_ss = d->dk_ss; p.dk_hs = d->dk_hs;
  p.qm = make_map(d->q_nseg, d->q_seg_len, d->q_seg_pos);
  p.km = make_map(d->k_nseg, d->k_seg_len, d->k_seg_pos);
  p.hq = d->hq; p.hkv = d->hkv; p.group = d->hq / d->hkv;
  p.causal = d->causal;
  p.dkv_accumulate = d->dkv_accumulate;
  p.scale = d->scale;
  p.scale_log2 = d->scale * 1.4426950408889634f;
  return p;
}

ra_status ring_attn_step_fwd(const ra_step_desc* d, const void* q, const void* k, const void* v,
                             float* o_step, float* lse_step, ra_stream_t stream) {
  ra_status st = ra_validate_step(d, 0);
  if (st != RA_OK) return st;
  const int64_t lq = (int64_t)d->q_nseg * d->q_seg_len;
  const int64_t lk = (int64_t)d->k_nseg * d->k_seg_len;
  if (lq == 0) return RA_OK;
  if (!q || !o_step || !lse_step) return RA_EINVAL;
  if (lk > 0 && (!k || !v)) return RA_EINVAL;
  if (!aligned16(q) || !aligned16(o_step) || !aligned16(lse_step)) return RA_EALIGN;
  if (lk > 0 && (!aligned16(k) || !aligned16(v))) return RA_EALIGN;
  StepParams p = make_params(d);
  p.q = q; p.k = k; p.v = v; p.o = o_step; p.lse_out = lse_step;
  return from_hip(launch_step_fwd(p, d->dtype, d->head_dim, (hipStream_t)stream));
}

ra_status ring_attn_step_fwd_merge(const ra_step_desc* d, const void* q, const void* k,
                                   const void* v, float* o_acc, float* lse_acc,
                                   ra_stream_t stream) {
  ra_status st = ra_validate_step(d, 0);
  if (st != RA_OK) return st;
  const int64_t lq = (int64_t)d->q_nseg * d->q_seg_len;
  const int64_t lk = (int64_t)d->k_nseg * d->k_seg_len;
  if (lq == 0 || lk == 0) return RA_OK;  // an empty chunk leaves the accumulators as they are
  if (!q || !k || !v || !o_acc || !lse_acc) return RA_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o_acc) || !aligned16(lse_acc))
    return RA_EALIGN;
  StepParams p = make_params(d);
  p.q = q; p.k = k; p.v = v; p.o = o_acc; p.lse_out = lse_acc;
  p.merge = 1;
  return from_hip(launch_step_fwd(p, d->dtype, d->head_dim, (hipStream_t)stream));
}

// the query side, the key/value strides and the scale of every chunk's
// descriptor must be those of the first
static bool same_query_side(const ra_step_desc* a, const ra_step_desc* b) {
  if (a->dtype != b->dtype || a->head_dim != b->head_dim || a->hq != b->hq || a->hkv != b->hkv)
    return false;
  if (a->q_nseg != b->q_nseg || a->q_seg_len != b->q_seg_len) return false;
  for (int i = 0; i < a->q_nseg; ++i)
    if (a->q_seg_pos[i] != b->q_seg_pos[i]) return false;
  return a->causal == b->causal && a->scale == b->scale && a->q_ss == b->q_ss &&
         a->q_hs == b->q_hs && a->k_ss == b->k_ss && a->k_hs == b->k_hs && a->v_ss == b->v_ss &&
         a->v_hs == b->v_hs && a->o_ss == b->o_ss && a->o_hs == b->o_hs;
}

ra_status ring_attn_fwd_chunks(const ra_step_desc* descs, int32_t n, const void* q,
                               const void* const* k, const void* const* v, float* o, float* lse,
                               ra_stream_t stream) {
  if (!descs || n < 1 || !k || !v) return RA_EINVAL;
  if (n > kMaxChunks) return RA_EUNSUPPORTED;
  for (int i = 0; i < n; ++i) {
    const ra_status st = ra_validate_step(&descs[i], 0);
    if (st != RA_OK) return st;
    if (!same_query_side(&descs[0], &descs[i])) return RA_EINVAL;
  }
  const ra_step_desc* d0 = &descs[0];
  if (d0->dtype != RA_BF16) return RA_EUNSUPPORTED;  // the MFMA kernels only
  const int64_t lq = (int64_t)d0->q_nseg * d0->q_seg_len;
  if (lq == 0) return RA_OK;
  if (!q || !o || !lse) return RA_EINVAL;
  if (!aligned16(q) || !aligned16(o) || !aligned16(lse)) return RA_EALIGN;
  ChunkSet ch;
  memset(&ch, 0, sizeof(ch));
  for (int i = 0; i < n; ++i) {
    const ra_step_desc* d = &descs[i];
    if ((int64_t)d->k_nseg * d->k_seg_len == 0) continue;  // an empty chunk adds nothing
    if (!k[i] || !v[i]) return RA_EINVAL;
    if (!aligned16(k[i]) || !aligned16(v[i])) return RA_EALIGN;
    ch.k[ch.n] = k[i];
    ch.v[ch.n] = v[i];
    ch.km[ch.n] = make_map(d->k_nseg, d->k_seg_len, d->k_seg_pos);
    ++ch.n;
  }
  StepParams p = make_params(d0);
  p.q = q; p.o = o; p.lse_out = lse;
  return from_hip(launch_fwd_chunks(p, ch, d0->head_dim, (hipStream_t)stream));
}

ra_status ring_attn_bwd_chunks(const ra_step_desc* descs, int32_t n, const void* q,
                               const void* const* k, const void* const* v, const void* dout,
                               const float* lse, const float* delta, float* dq, float* const* dk,
                               float* const* dv, ra_stream_t stream) {
  if (!descs || n < 1 || !k || !v || !dk || !dv) return RA_EINVAL;
  if (n > kMaxChunks) return RA_EUNSUPPORTED;
  for (int i = 0; i < n; ++i) {
    const ra_status st = ra_validate_step(&descs[i], 1);
    if (st != RA_OK) return st;
    const ra_step_desc* d = &descs[i];
    if (!same_query_side(&descs[0], d) || d->do_ss != descs[0].do_ss ||
        d->do_hs != descs[0].do_hs || d->dk_ss != descs[0].dk_ss || d->dk_hs != descs[0].dk_hs)
      return RA_EINVAL;
  }
  const ra_step_desc* d0 = &descs[0];
  if (d0->dtype != RA_BF16) return RA_EUNSUPPORTED;  // the MFMA kernels only
  const int64_t lq = (int64_t)d0->q_nseg * d0->q_seg_len;
  if (lq > 0) {
    if (!q || !dout || !lse || !delta || !dq) return RA_EINVAL;
    if (!aligned16(q) || !aligned16(dout) || !aligned16(lse) || !aligned16(delta) ||
        !aligned16(dq))
      return RA_EALIGN;
  }
  ChunkSet ch;
  memset(&ch, 0, sizeof(ch));
  float* dks[kMaxChunks];
  float* dvs[kMaxChunks];
  int32_t acc[kMaxChunks];
  for (int i = 0; i < n; ++i) {
    const ra_step_desc* d = &descs[i];
    if ((int64_t)d->k_nseg * d->k_seg_len == 0) continue;  // an empty chunk adds nothing
    if (!k[i] || !v[i] || !dk[i] || !dv[i]) return RA_EINVAL;
    if (!aligned16(k[i]) || !aligned16(v[i]) || !aligned16(dk[i]) || !aligned16(dv[i]))
      return RA_EALIGN;
    ch.k[ch.n] = k[i];
    ch.v[ch.n] = v[i];
    ch.km[ch.n] = make_map(d->k_nseg, d->k_seg_len, d->k_seg_pos);
    dks[ch.n] = dk[i];
    dvs[ch.n] = dv[i];
    acc[ch.n] = d->dkv_accumulate;
    ++ch.n;
  }
  StepParams p = make_params(d0);
  p.q = q; p.dout = dout; p.lse_in = lse; p.delta = delta; p.o = dq;
  return from_hip(launch_bwd_chunks(p, ch, dks, dvs, acc, d0->head_dim, (hipStream_t)stream));
}

ra_status ring_attn_step_bwd(const ra_step_desc* d, const void* q, const void* k, const void* v,
                             const void* dout, const float* lse, const float* delta,
                             float* dq_acc, float* dk_acc, float* dv_acc, ra_stream_t stream) {
  ra_status st = ra_validate_step(d, 1);
  if (st != RA_OK) return st;
  const int64_t lq = (int64_t)d->q_nseg * d->q_seg_len;
  const int64_t lk = (int64_t)d->k_nseg * d->k_seg_len;
  if (lk == 0) return RA_OK;
  if (!k || !v || !dk_acc || !dv_acc) return RA_EINVAL;
  if (!aligned16(k) || !aligned16(v) || !aligned16(dk_acc) || !aligned16(dv_acc)) return RA_EALIGN;
  if (lq > 0) {
    if (!q || !dout || !lse || !delta || !dq_acc) return RA_EINVAL;
    if (!aligned16(q) || !aligned16(dout) || !aligned16(lse) || !aligned16(delta) ||
        !aligned16(dq_acc))
      return RA_EALIGN;
  }
  StepParams p = make_params(d);
  p.q = q; p.k = k; p.v = v; p.dout = dout; p.lse_in = lse; p.delta = delta;
  p.o = dq_acc; p.dk = dk_acc; p.dv = dv_acc;
  return from_hip(launch_step_bwd(p, d->dtype, d->head_dim, (hipStream_t)stream));
}

ra_status lse_merge(int64_t rows, int32_t hq, int32_t head_dim, int64_t row_begin,
                    int64_t row_count, float* o_acc, float* lse_acc, const float* o_step,
                    const float* lse_step, ra_stream_t stream) {
  if (rows < 0 || hq < 1) return RA_EINVAL;
  if (row_begin < 0 || row_count < 0 || row_begin > rows || row_count > rows - row_begin)
    return RA_EINVAL;
  if (head_dim != 64 && head_dim != 128) return RA_EUNSUPPORTED;
  if (rows * (int64_t)hq > (int64_t)UINT32_MAX) return RA_EUNSUPPORTED;  // 32-bit row index
  if (row_count == 0) return RA_OK;
  if (!o_acc || !lse_acc || !o_step || !lse_step) return RA_EINVAL;
  if (!aligned16(o_acc) || !aligned16(o_step) || !aligned16(lse_acc) || !aligned16(lse_step))
    return RA_EALIGN;
  return from_hip(launch_lse_merge(rows, hq, head_dim, row_begin, row_count, o_acc, lse_acc,
                                   o_step, lse_step, (hipStream_t)stream));
}

ra_status ra_bwd_delta(int64_t rows, int32_t hq, int32_t head_dim, int32_t dtype, const float* o,
                       const void* dout, float* delta, void* o_out, ra_stream_t stream) {
  if (rows < 0 || hq < 1) return RA_EINVAL;
  if (dtype != RA_BF16 && dtype != RA_F32) return RA_EINVAL;
  if (head_dim != 64 && head_dim != 128) return RA_EUNSUPPORTED;
  if (rows * (int64_t)hq > (int64_t)UINT32_MAX) return RA_EUNSUPPORTED;  // 32-bit row index
  if (rows == 0) return RA_OK;
  if (!o || !dout || !delta) return RA_EINVAL;
  if (!aligned16(o) || !aligned16(dout) || !aligned16(delta) || (o_out && !aligned16(o_out)))
    return RA_EALIGN;
  return from_hip(launch_bwd_delta(rows, hq, head_dim, dtype, o, dout, delta, o_out,
                                   (hipStream_t)stream));
}

ra_status head_permute(const void* src, void* dst, int64_t s, int32_t h, int32_t d, int32_t p,
                       int32_t elem_bytes_, int32_t inverse, ra_stream_t stream) {
  if (s < 0 || h < 1 || d < 1 || p < 1) return RA_EINVAL;
  if (elem_bytes_ != 2 && elem_bytes_ != 4) return RA_EINVAL;
  if (inverse != 0 && inverse != 1) return RA_EINVAL;
  if (h % p != 0) return RA_EINVAL;  // every destination needs whole heads
  if (p > 65535) return RA_EUNSUPPORTED;  // one grid row per head group
  if (((int64_t)(h / p) * d * elem_bytes_) % 16 != 0) return RA_EALIGN;
  if (s == 0) return RA_OK;
  if (!src || !dst) return RA_EINVAL;
  if (!aligned16(src) || !aligned16(dst)) return RA_EALIGN;
  const int64_t bytes = s * (int64_t)h * d * elem_bytes_;
  const char* a = (const char*)src;
  const char* b = (const char*)dst;
  if (a < b + bytes && b < a + bytes) return RA_EINVAL;  // overlapping buffers
  return from_hip(launch_head_permute(src, dst, s, h, d, p, elem_bytes_, inverse,
                                      (hipStream_t)stream));
}

ra_status ra_fill_f32(float* dst, int64_t n, float value, ra_stream_t stream) {
  if (n < 0) return RA_EINVAL;
  if (n == 0) return RA_OK;
  if (!dst) return RA_EINVAL;
  if (!aligned16(dst)) return RA_EALIGN;
  return from_hip(launch_fill_f32(dst, n, value, (hipStream_t)stream));
}

ra_status ra_zigzag_segments(int64_t S, int32_t P, int32_t rank, int64_t* seg_pos_out,
                             int64_t* seg_len_out) {
  if (S < 0 || P < 1 || rank < 0 || rank >= P || !seg_pos_out || !seg_len_out) return RA_EINVAL;
  if (S % (2 * (int64_t)P) != 0) return RA_EINVAL;
  const int64_t b = S / (2 * (int64_t)P);
  seg_pos_out[0] = (int64_t)rank * b;
  seg_pos_out[1] = (int64_t)(2 * P - 1 - rank) * b;
  *seg_len_out = b;
  return RA_OK;
}

ra_status ra_zigzag_positions(int64_t S, int32_t P, int32_t rank, int64_t* pos_out) {
  int64_t seg[2], b;
  ra_status st = ra_zigzag_segments(S, P, rank, seg, &b);
  if (st != RA_OK) return st;
  if (!pos_out) return RA_EINVAL;
  for (int64_t i = 0; i < b; ++i) {
    pos_out[i] = seg[0] + i;
    pos_out[b + i] = seg[1] + i;
  }
  return RA_OK;
}

ra_status ra_double_ring_order(int32_t inner, int32_t outer, int32_t rank, int32_t* chunk_out) {
  if (inner < 1 || outer < 1 || !chunk_out) return RA_EINVAL;
  const int64_t P = (int64_t)inner * outer;
  if (P > (1 << 20) || rank < 0 || rank >= P) return RA_EINVAL;
  const int32_t g = rank / inner, l = rank % inner;
  for (int32_t o = 0; o < outer; ++o) {
    const int32_t src_group = ((g - o) % outer + outer) % outer;
    for (int32_t i = 0; i < inner; ++i) {
      const int32_t src_local = ((l - i) % inner + inner) % inner;
      chunk_out[o * inner + i] = src_group * inner + src_local;
    }
  }
  return RA_OK;
}

}  // extern "C"
