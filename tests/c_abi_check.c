/* The C ABI used from plain C99 (no C++, no Python): host-only calls and the
 * argument checks of the device calls, which return before any device work.
 * Built and run by tests/test_c_abi.py; prints "ok" and exits 0 on success. */
#include <stdio.h>
#include <string.h>

#include "ring_attn.h"

#define CHECK(c)                                              \
  do {                                                        \
    if (!(c)) {                                               \
      fprintf(stderr, "failed: %s (line %d)\n", #c, __LINE__); \
      return 1;                                               \
    }                                                         \
  } while (0)

static ra_step_desc good_desc(void) {
  ra_step_desc d;
  memset(&d, 0, sizeof(d));
  d.dtype = RA_BF16;
  d.head_dim = 128;
  d.hq = 8;
  d.hkv = 2;
  d.q_nseg = d.k_nseg = 2;
  d.q_seg_len = d.k_seg_len = 64;
  d.q_seg_pos[0] = 64;
  d.q_seg_pos[1] = 384;
  d.k_seg_pos[0] = 0;
  d.k_seg_pos[1] = 448;
  d.causal = 1;
  d.scale = 0.08838834764831845f;
  d.q_ss = 8 * 128, d.q_hs = 128;
  d.k_ss = 2 * 128, d.k_hs = 128;
  d.v_ss = 2 * 128, d.v_hs = 128;
  d.o_ss = 8 * 128, d.o_hs = 128;
  d.do_ss = 8 * 128, d.do_hs = 128;
  d.dk_ss = 2 * 128, d.dk_hs = 128;
  return d;
}

int main(void) {
  /* paired blocks: S = 512, P = 4, b = 64; rank 1 holds blocks 1 and 6 */
  int64_t pos[128], seg[2], seg_len = 0;
  int i, t;
  CHECK(ra_zigzag_positions(512, 4, 1, pos) == RA_OK);
  for (i = 0; i < 64; ++i) CHECK(pos[i] == 64 + i && pos[64 + i] == 384 + i);
  CHECK(ra_zigzag_segments(512, 4, 1, seg, &seg_len) == RA_OK);
  CHECK(seg[0] == 64 && seg[1] == 384 && seg_len == 64);
  CHECK(ra_zigzag_positions(500, 4, 1, pos) == RA_EINVAL);  /* S % 2P != 0 */
  CHECK(ra_zigzag_positions(512, 4, 4, pos) == RA_EINVAL);  /* rank out of range */

  /* double ring 4 x 2, rank 5 = group 1, lane 1 */
  {
    int32_t ch[8];
    CHECK(ra_double_ring_order(4, 2, 5, ch) == RA_OK);
    for (t = 0; t < 8; ++t) {
      const int o = t / 4, l = t % 4;
      CHECK(ch[t] == ((1 - o + 2) % 2) * 4 + ((1 - l + 4) % 4));
    }
  }

  /* descriptor checks */
  {
    ra_step_desc d = good_desc();
    CHECK(ra_validate_step(&d, 1) == RA_OK);
    d.head_dim = 96;
    CHECK(ra_validate_step(&d, 0) == RA_EUNSUPPORTED);
    d = good_desc();
    d.hq = 7;  /* hq % hkv != 0 */
    CHECK(ra_validate_step(&d, 0) == RA_EINVAL);
    CHECK(ra_validate_step(NULL, 0) == RA_EINVAL);
  }

  /* device calls refuse bad arguments before touching the device */
  {
    ra_step_desc d = good_desc();
    const void* ks[2] = {0, 0};
    float* dks[2] = {0, 0};
    CHECK(ring_attn_step_fwd(NULL, 0, 0, 0, 0, 0, 0) == RA_EINVAL);
    d.head_dim = 96;
    CHECK(ring_attn_step_bwd(&d, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0) == RA_EUNSUPPORTED);
    d = good_desc();
    CHECK(ring_attn_fwd_chunks(&d, 0, 0, ks, ks, 0, 0, 0) == RA_EINVAL);  /* n = 0 */
    CHECK(ring_attn_bwd_chunks(&d, RA_MAX_CHUNKS + 1, 0, ks, ks, 0, 0, 0, 0, dks, dks, 0) ==
          RA_EUNSUPPORTED);
    CHECK(lse_merge(64, 8, 96, 0, 64, 0, 0, 0, 0, 0) == RA_EUNSUPPORTED);
  }

  CHECK(strlen(ra_status_str(RA_EALIGN)) > 0);
  printf("ok\n");
  return 0;
}
