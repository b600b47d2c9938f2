/*
 * ring_attn.h -- C ABI of libringattn.so: one GPU's share of context-parallel
 * (ring) causal attention with grouped-query heads, for AMD MI355X (gfx950).
 *
 * The method (sources are cited by page title and section):
 *   - "LoongTrain: Efficient Training of Long-Sequence LLMs with Head-Context
 *     Parallelism", abstract: 2D-Attention combines head-parallel and
 *     context-parallel attention; the context ring is run as
 *     Double-Ring-Attention.
 *   - "Guide to LoongTrain: 2D Head-Context Parallelism for LLMs":
 *       "The Communication Overhead and Causal Imbalance of Ring Attention":
 *         each rank keeps its query chunk Q_i, receives (K_j, V_j) from its ring
 *         predecessor at every step and attends to it; a query at position p
 *         sees a key at position p' iff p' <= p.
 *       "2. Paired-Block Allocation for Causal Load Balancing": the sequence is
 *         cut into 2P blocks and rank r holds blocks r and 2P-1-r.
 *       "The Scalability Limits of DeepSpeed Ulysses": the head all-to-all
 *         (S/P, H) <-> (S, H/P), and P_ulysses <= H_kv.
 *       "Step 3" reference code: scale = 1/sqrt(head_dim), softmax(QK^T scale) V.
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE pointers (HIP global memory) owned by the
 *     caller. The library allocates no memory and keeps no mutable global
 *     state; calls on different streams are independent.
 *   - Every argument is validated on the host before anything is enqueued. On a
 *     bad argument the call returns RA_EINVAL / RA_EUNSUPPORTED / RA_EALIGN and
 *     enqueues nothing. A failed kernel launch returns RA_EDEVICE.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; 0 = the
 *     null stream); no call synchronises. Nothing throws or aborts.
 *   - Floating-point outputs are fp32. Logs are natural logs.
 *   - Layouts are token-major: a [rows][heads][d] tensor is addressed as
 *     base + row*seq_stride + head*head_stride + x, the last dimension
 *     contiguous; strides are in ELEMENTS. LSE and D vectors are [heads][rows],
 *     contiguous (head stride = rows).
 *   - Pointers must be 16-byte aligned; seq/head strides must keep every row
 *     16-byte aligned (else RA_EALIGN).
 */
#ifndef RING_ATTN_H
#define RING_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RA_OK = 0,
  RA_EINVAL = 1,        /* malformed arguments (shapes, ranks, null pointers) */
  RA_EUNSUPPORTED = 2,  /* well-formed but not built (e.g. head_dim 96)        */
  RA_EALIGN = 3,        /* pointer or stride alignment                         */
  RA_EDEVICE = 4        /* the HIP runtime refused a launch                    */
} ra_status;

typedef enum { RA_BF16 = 0, RA_F32 = 1 } ra_dtype;

/* most chunks one ring_attn_fwd_chunks / ring_attn_bwd_chunks call takes */
#define RA_MAX_CHUNKS 32

typedef void* ra_stream_t; /* a hipStream_t */

/*
 * One ring step: local query rows against one KV chunk.
 *
 * Rows of the query buffer (and of the KV buffer) are 1 or 2 runs ("segments")
 * of consecutive global positions: with the paired-block layout a chunk of
 * rank r is [block r ; block 2P-1-r], i.e. nseg = 2, seg_len = b = S/(2P),
 * seg_pos = {r*b, (2P-1-r)*b}. Row i of the buffer has position
 * seg_pos[i / seg_len] + i % seg_len; lq = q_nseg*q_seg_len, lk = k_nseg*k_seg_len.
 *
 * Query head h uses KV head h / (hq/hkv).
 */
typedef struct ra_step_desc {
  int32_t dtype;        /* ra_dtype of q, k, v, dout                               */
  int32_t head_dim;     /* d: 64 or 128                                            */
  int32_t hq, hkv;      /* local query / KV heads, hq % hkv == 0                   */
  int32_t q_nseg, k_nseg;          /* 1 or 2                                       */
  int64_t q_seg_len, k_seg_len;    /* >= 0; a zero-row call is a no-op             */
  int64_t q_seg_pos[2], k_seg_pos[2]; /* global position of each segment's row 0   */
  int32_t causal;       /* 1: key visible iff pos_k <= pos_q; 0: all keys visible  */
  float scale;          /* softmax scale > 0, normally 1/sqrt(head_dim)            */
  int64_t q_ss, q_hs;   /* q    [lq][hq][d]                                        */
  int64_t k_ss, k_hs;   /* k    [lk][hkv][d]                                       */
  int64_t v_ss, v_hs;   /* v    [lk][hkv][d]                                       */
  int64_t o_ss, o_hs;   /* fp32 [lq][hq][d]: o_step (fwd) and dq_acc (bwd)         */
  int64_t do_ss, do_hs; /* dout [lq][hq][d] (bwd)                                  */
  int64_t dk_ss, dk_hs; /* fp32 [lk][hkv][d]: dk_acc and dv_acc (bwd)              */
  int32_t dkv_accumulate; /* bwd: 1 = add into dk_acc/dv_acc, 0 = overwrite them   */
  int32_t reserved;
} ra_step_desc;

/*
 * ring_attn_step_fwd -- attention of the local queries against one KV chunk
 * (the per-step computation of the ring: "Guide to LoongTrain", "The
 * Communication Overhead and Causal Imbalance of Ring Attention").
 *
 * For query head h, row i, with s_ij = scale * q_i . k_j over the chunk's
 * visible keys j:  lse_step[h][i] = ln sum_j exp(s_ij)  and
 * o_step[i][h][:] = sum_j exp(s_ij - lse_step[h][i]) v_j.
 * A row with no visible key gets o_step = 0 and lse_step = -inf.
 * Writes every one of the lq rows of o_step and lse_step (no accumulation).
 * q, k, v: bf16 or fp32 per desc->dtype. MFMA bf16 with fp32 accumulation for
 * bf16; fp32 arithmetic for fp32.
 */
ra_status ring_attn_step_fwd(const ra_step_desc* desc, const void* q, const void* k,
                             const void* v, float* o_step, float* lse_step,
                             ra_stream_t stream);

/*
 * ring_attn_step_fwd_merge -- ring_attn_step_fwd followed by lse_merge of its
 * result into the running (o_acc, lse_acc), in one kernel: the step's rows are
 * folded into the accumulators in the kernel's epilogue (the merge formula of
 * lse_merge, below) and never written out, which saves the step's O_step and
 * LSE_step round trip through memory.
 * o_acc: fp32 with desc's o strides; lse_acc: fp32 [hq][lq]; both updated in
 * place (initialise them as for lse_merge: lse_acc = -inf, o_acc = 0, or with a
 * first step). A row with no visible key in this chunk is left unchanged; an
 * empty chunk (lk == 0) launches nothing. Same inputs, arithmetic and errors as
 * ring_attn_step_fwd; calls that overlap on the same accumulators race.
 */
ra_status ring_attn_step_fwd_merge(const ra_step_desc* desc, const void* q, const void* k,
                                   const void* v, float* o_acc, float* lse_acc,
                                   ra_stream_t stream);

/*
 * ring_attn_fwd_chunks -- the forward of all n ring steps of this share in one
 * launch: ring_attn_step_fwd of chunk 0 folded with chunks 1 .. n-1 as
 * ring_attn_step_fwd_merge folds them ("Guide to LoongTrain", "The
 * Communication Overhead and Causal Imbalance of Ring Attention": each rank
 * attends its queries to every KV chunk), for a GPU that holds every chunk (the
 * one-GPU virtual ring). The running max, sum and output stay in registers from
 * one chunk to the next and O, LSE are written once, so no partial result goes
 * through memory; the softmax is the same, its rounding differs from the
 * per-step path's (no intermediate normalisation).
 * descs: n descriptors, chunk i's key side in descs[i]; every other field
 * (dtype, head_dim, heads, query segments, causal, scale, q/k/v/o strides)
 * must equal descs[0]'s (RA_EINVAL otherwise). k, v: host arrays of n device
 * pointers (chunk i's K and V). o: fp32 [lq][hq][d] (descs[0]'s o strides),
 * lse: fp32 [hq][lq], both written (rows with no visible key anywhere: O = 0,
 * LSE = -inf). 1 <= n <= RA_MAX_CHUNKS (RA_EUNSUPPORTED beyond); bf16 only
 * (RA_EUNSUPPORTED for fp32). Chunks with lk == 0 are skipped.
 */
ra_status ring_attn_fwd_chunks(const ra_step_desc* descs, int32_t n, const void* q,
                               const void* const* k, const void* const* v, float* o,
                               float* lse, ra_stream_t stream);

/*
 * ring_attn_bwd_chunks -- the backward of all n ring steps: dQ of every chunk
 * in one launch, summed in registers over the chunks and written once (no
 * read-modify-write of dQ per step), then dK/dV of every chunk in a second
 * launch, each chunk's exactly as ring_attn_step_bwd computes them (bit for
 * bit from the same LSE and D). Same arithmetic as ring_attn_step_bwd over the
 * chunks (dQ's summation order over chunks differs from accumulating it step
 * by step); for a GPU that holds every chunk, like ring_attn_fwd_chunks.
 * A chunk with lk == 0 is skipped (its pointers are not read, its dK/dV left
 * as they are); with lq == 0, dq, q, dout, lse and delta are not read and
 * dK/dV are written as zeros (left as they are when dkv_accumulate).
 * descs: n descriptors (chunk i's key side and dkv_accumulate in descs[i]; all
 * other fields, including the dout and dK strides, equal to descs[0]'s).
 * k, v, dk, dv: host arrays of n device pointers (chunk i's K, V and its dK,
 * dV outputs, fp32 with the dk strides; added to when dkv_accumulate).
 * dq: fp32 with descs[0]'s o strides, WRITTEN (not accumulated). lse, delta:
 * the final LSE and D, fp32 [hq][lq]. 1 <= n <= RA_MAX_CHUNKS; bf16 only.
 * Errors as for ring_attn_fwd_chunks and ring_attn_step_bwd.
 */
ra_status ring_attn_bwd_chunks(const ra_step_desc* descs, int32_t n, const void* q,
                               const void* const* k, const void* const* v, const void* dout,
                               const float* lse, const float* delta, float* dq,
                               float* const* dk, float* const* dv, ra_stream_t stream);

/*
 * ring_attn_step_bwd -- one step's share of the attention gradient, driven by
 * the FINAL log-sum-exp and D of the rows (saved-LSE recompute).
 *
 * The pages give no backward formula (the LoongTrain abstract only names
 * Selective Checkpoint++ recomputation). The reading taken: the exact gradient
 * of sum(dout * O) over this share's rows, restricted to the chunk's keys,
 * with D from the final fp32 O; P and dS are rounded to bf16 (nearest even)
 * before they enter a bf16 product, and dK/dV are this share's contribution
 * only (a multi-GPU ring would sum them over the ranks).
 *
 * P_ij = exp(s_ij - lse[h][i]) on visible pairs, dP_ij = dout_i . v_j,
 * dS_ij = P_ij (dP_ij - delta[h][i]);
 *   dq_acc[i][h]  += scale * sum_j dS_ij k_j          (always accumulates)
 *   dk_acc[j][g]  (+)= scale * sum_{h in g, i} dS_ij q_i
 *   dv_acc[j][g]  (+)= sum_{h in g, i} P_ij dout_i    (per desc->dkv_accumulate)
 * dq_acc must be initialised by the caller (e.g. ra_fill_f32 to 0). Every
 * element of dq_acc, dk_acc and dv_acc is read-modify-written by one thread,
 * so results are deterministic; calls that overlap on the same accumulators
 * race. bf16 runs two kernels (dQ; dK and dV) on `stream`, in that order.
 */
ra_status ring_attn_step_bwd(const ra_step_desc* desc, const void* q, const void* k,
                             const void* v, const void* dout, const float* lse,
                             const float* delta, float* dq_acc, float* dk_acc,
                             float* dv_acc, ra_stream_t stream);

/*
 * lse_merge -- fold one step's partial result into the running one: the
 * "online-softmax rescaling" by which partial outputs over disjoint key sets
 * are merged. The pages print no formula for it; this is the max-shifted
 * log-sum-exp rescale (the reading taken):
 *   m = max(La, Ls); if m == -inf the row stays (O unchanged, L = -inf), else
 *   L = m + ln(e^(La-m) + e^(Ls-m)), O = e^(La-L) Oa + e^(Ls-L) Os.
 * o_acc, o_step: fp32 [rows][hq][d] contiguous; lse_acc, lse_step: fp32
 * [hq][rows]. Only rows [row_begin, row_begin + row_count) are read and
 * updated (in place), e.g. the rows a ring step gave any visible key: with
 * paired blocks, a chunk later than the rank's own is seen by block B only.
 * RA_EINVAL unless 0 <= row_begin <= rows and 0 <= row_count <= rows - row_begin;
 * RA_EUNSUPPORTED for rows * hq >= 2^32; row_count == 0 is a no-op.
 */
ra_status lse_merge(int64_t rows, int32_t hq, int32_t head_dim, int64_t row_begin,
                    int64_t row_count, float* o_acc, float* lse_acc, const float* o_step,
                    const float* lse_step, ra_stream_t stream);

/*
 * ra_bwd_delta -- backward preprocess of the merged forward result. The pages
 * give no formula; this is the row term of the exact softmax gradient (the same
 * reading as ring_attn_step_bwd), computed from the final fp32 O:
 *   delta[h][i] = sum_x dout[i][h][x] * o[i][h][x]
 * and, if o_out != NULL, o_out = o rounded to bf16 (nearest even).
 * o: fp32 [rows][hq][d]; dout: dtype [rows][hq][d]; o_out: bf16 [rows][hq][d];
 * all contiguous. delta: fp32 [hq][rows]. RA_EUNSUPPORTED for rows * hq >= 2^32.
 */
ra_status ra_bwd_delta(int64_t rows, int32_t hq, int32_t head_dim, int32_t dtype,
                       const float* o, const void* dout, float* delta, void* o_out,
                       ra_stream_t stream);

/*
 * head_permute -- the local layout change of the head all-to-all ("Guide to
 * LoongTrain", "The Scalability Limits of DeepSpeed Ulysses": (S/P, H) ->
 * (S, H/P) before attention, back after it).
 * inverse == 0: src [s][h][d] -> dst [p][s][h/p][d], dst[q][t][j][x] =
 *               src[t][q*(h/p) + j][x] (destination q receives head group q);
 * inverse == 1: the exact inverse (src is [p][s][h/p][d]).
 * A bit copy of elem_bytes (2 or 4) wide elements; both contiguous;
 * requires h % p == 0 and (h/p)*d*elem_bytes a multiple of 16 (RA_EALIGN
 * otherwise). src and dst must not overlap. p > 65535 returns RA_EUNSUPPORTED.
 */
ra_status head_permute(const void* src, void* dst, int64_t s, int32_t h, int32_t d,
                       int32_t p, int32_t elem_bytes, int32_t inverse,
                       ra_stream_t stream);

/* ra_fill_f32 -- dst[0..n) = value (accumulator initialisation). */
ra_status ra_fill_f32(float* dst, int64_t n, float value, ra_stream_t stream);

/* ---- host-only helpers: no device work, safe without a GPU ---------------- */

/*
 * ra_zigzag_positions -- global positions of the 2b rows of ring chunk `rank`
 * ("2. Paired-Block Allocation for Causal Load Balancing"): b = S/(2P);
 * pos_out[i] = rank*b + i and pos_out[b+i] = (2P-1-rank)*b + i for i < b.
 * pos_out has room for 2b values. RA_EINVAL unless S % (2P) == 0, 0 <= rank < P.
 */
ra_status ra_zigzag_positions(int64_t S, int32_t P, int32_t rank, int64_t* pos_out);

/*
 * ra_zigzag_segments -- the same map as segment descriptors for ra_step_desc:
 * seg_pos_out[0] = rank*b, seg_pos_out[1] = (2P-1-rank)*b, *seg_len_out = b.
 */
ra_status ra_zigzag_segments(int64_t S, int32_t P, int32_t rank, int64_t* seg_pos_out,
                             int64_t* seg_len_out);

/*
 * ra_double_ring_order -- chunk visited by `rank` at each of the P = inner*outer
 * steps of the double ring (abstract of the LoongTrain paper; "3. Double-Ring
 * Asynchronous Communication Pipeline"): K/V move one hop from the predecessor
 * per step; ranks form groups of `inner` consecutive ids, the inner ring turns
 * inside a group and the outer ring advances one group every `inner` steps:
 * with t = o*inner + i and rank = g*inner + l,
 * chunk_out[t] = ((g-o) mod outer)*inner + ((l-i) mod inner).
 */
ra_status ra_double_ring_order(int32_t inner, int32_t outer, int32_t rank,
                               int32_t* chunk_out);

/*
 * ra_validate_step -- the host-side check that ring_attn_step_fwd/_bwd run
 * before enqueueing (exported so it can be exercised without a GPU).
 * for_bwd selects the backward's extra stride checks.
 */
ra_status ra_validate_step(const ra_step_desc* desc, int32_t for_bwd);

/* Static string naming a status code. */
const char* ra_status_str(ra_status s);

#ifdef __cplusplus
}
#endif

#endif /* RING_ATTN_H */
