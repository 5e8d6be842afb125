// Host harness of the C ABI's validation layer (include/rssm.h), run under AddressSanitizer and
// UndefinedBehaviorSanitizer without a GPU: configuration checks over a grid of valid and
// invalid sizes, buffer sizing and ring offsets, and every entry point with rejected arguments
// (nothing may be launched) and with an empty batch.  Prints "ok" and exits 0 on success.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "rssm.h"

extern "C" int rssm_stub_launches;

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond);        \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

static rssm_config cfg(int kind, int B, int H, int G, int P, int N, int L, int T, int C, int dt, int rc) {
  rssm_config c;
  c.kind = kind; c.batch = B; c.n_heads = H; c.n_qk_heads = G; c.dv = P; c.dk = N;
  c.L = L; c.t_max = T; c.capacity = C; c.in_dtype = dt; c.read_copy = rc;
  return c;
}

int main() {
  // --- configurations: a grid of sizes, each checked for internal consistency when accepted
  const int kinds[] = {RSSM_KIND_MAMBA2, RSSM_KIND_GDN, RSSM_KIND_KDA, 3, -1};
  const int dks[] = {0, 16, 32, 48, 64, 128, 256, 512};
  const int dvs[] = {-1, 0, 1, 17, 64, 128, 512, 513, 1 << 20};
  int accepted = 0;
  for (int kind : kinds)
    for (int N : dks)
      for (int P : dvs)
        for (int T : {0, 1, 4, 8, 9})
          for (int C : {1, 16, 19, 32, 33}) {
            rssm_config c = cfg(kind, 3, 4, 2, P, N, 16, T, C, RSSM_DTYPE_BF16, RSSM_READ_FP8);
            const int r = rssm_check_config(&c);
            rssm_buffer_sizes sz;
            int64_t off[5];
            EXPECT(rssm_sizes(&c, &sz) == r);
            EXPECT(rssm_ring_offsets(&c, off) == r);
            if (r != RSSM_OK) continue;
            ++accepted;
            EXPECT(kind >= 0 && kind <= 2 && T >= 1 && T <= 8 && C >= 16 + T - 1 && C <= 32);
            EXPECT(sz.s_ckpt == (size_t)3 * 4 * P * N * 4);
            for (int i = 0; i < 5; ++i) EXPECT(off[i] % 256 == 0 && off[i] >= 0 && (size_t)off[i] <= sz.ring);
            for (int i = 0; i < 4; ++i) EXPECT(off[i] <= off[i + 1]);
          }
  EXPECT(accepted > 0);
  rssm_config bad = cfg(RSSM_KIND_MAMBA2, 2, 3, 2, 16, 32, 16, 1, 16, RSSM_DTYPE_F32, RSSM_READ_NONE);
  EXPECT(rssm_check_config(&bad) == RSSM_E_SHAPE);                   // H % G != 0
  bad = cfg(RSSM_KIND_MAMBA2, -1, 4, 4, 16, 32, 16, 1, 16, RSSM_DTYPE_F32, RSSM_READ_NONE);
  EXPECT(rssm_check_config(&bad) == RSSM_E_SHAPE);
  bad = cfg(RSSM_KIND_MAMBA2, 2, 4, 4, 16, 32, 16, 1, 16, 7, RSSM_READ_NONE);
  EXPECT(rssm_check_config(&bad) == RSSM_E_DTYPE);
  bad = cfg(RSSM_KIND_MAMBA2, 2, 4, 4, 16, 32, 16, 1, 16, RSSM_DTYPE_F32, 9);
  EXPECT(rssm_check_config(&bad) == RSSM_E_DTYPE);
  bad = cfg(RSSM_KIND_MAMBA2, 1 << 20, 1 << 12, 1 << 12, 64, 128, 16, 1, 16, RSSM_DTYPE_BF16, RSSM_READ_NONE);
  EXPECT(rssm_check_config(&bad) == RSSM_E_SHAPE);                   // more than 2^30 tiles
  EXPECT(rssm_check_config(nullptr) == RSSM_E_NULL);
  EXPECT(rssm_sizes(nullptr, nullptr) == RSSM_E_NULL);

  // --- entry points: rejected arguments launch nothing
  rssm_config c = cfg(RSSM_KIND_GDN, 2, 4, 2, 64, 128, 16, 4, 19, RSSM_DTYPE_BF16, RSSM_READ_NONE);
  EXPECT(rssm_check_config(&c) == RSSM_OK);
  alignas(256) static unsigned char buf[1 << 16];
  char *p = (char *)buf;
  rssm_state st = {(float *)p, nullptr, nullptr, p, (int64_t *)p, (int64_t *)p, (int32_t *)p};
  rssm_state nul = st;
  nul.ring = nullptr;
  rssm_state mis = st;
  mis.s_ckpt = (float *)(p + 4);
  const void *in = p;
  float *y = (float *)p;
  const int32_t *iv = (const int32_t *)p;
  rssm_stub_launches = 0;
  EXPECT(rssm_decode_step(&c, &nul, in, in, in, in, in, y, 0) == RSSM_E_NULL);
  EXPECT(rssm_decode_step(&c, &mis, in, in, in, in, in, y, 0) == RSSM_E_ALIGN);
  EXPECT(rssm_decode_step(&c, &st, in, nullptr, in, in, in, y, 0) == RSSM_E_NULL);   // GDN needs beta
  EXPECT(rssm_decode_step(&c, &st, p + 1, in, in, in, in, y, 0) == RSSM_E_ALIGN);     // bf16 needs 2 bytes
  EXPECT(rssm_decode_step(nullptr, &st, in, in, in, in, in, y, 0) == RSSM_E_NULL);
  EXPECT(rssm_verify(&c, &st, 0, in, in, in, in, in, y, 0) == RSSM_E_RANGE);
  EXPECT(rssm_verify(&c, &st, 5, in, in, in, in, in, y, 0) == RSSM_E_RANGE);
  EXPECT(rssm_verify_tree(&c, &st, 4, nullptr, in, in, in, in, in, y, 0) == RSSM_E_NULL);
  EXPECT(rssm_verify_fold(&c, &st, 16, 9, nullptr, in, in, in, in, in, y, 0) == RSSM_E_RANGE);
  EXPECT(rssm_commit(&c, &st, iv, 9, 0) == RSSM_E_RANGE);
  EXPECT(rssm_commit(&c, &st, nullptr, 4, 0) == RSSM_E_NULL);
  EXPECT(rssm_commit_tree(&c, &st, iv, nullptr, iv, 4, 0) == RSSM_E_NULL);
  EXPECT(rssm_flush(&c, &st, -1, 0) == RSSM_E_RANGE);
  EXPECT(rssm_flush(&c, &nul, 16, 0) == RSSM_E_NULL);
  EXPECT(rssm_verify_snapshot(&c, nullptr, iv, 4, in, in, in, in, in, y, (int32_t *)p, 0) == RSSM_E_NULL);
  EXPECT(rssm_commit_snapshot(&c, (int32_t *)p, iv, 0, (int32_t *)p, 0) == RSSM_E_RANGE);
  EXPECT(rssm_decode_step_conventional(&c, (float *)(p + 4), in, in, in, in, in, y, 0) == RSSM_E_ALIGN);
  EXPECT(rssm_stream_copy(p, p + 16, 100, 0) == RSSM_E_ALIGN);
  EXPECT(rssm_init_state(&c, &mis, nullptr, 0) == RSSM_E_ALIGN);
  EXPECT(rssm_stub_launches == 0);

  // --- an empty batch enqueues nothing
  rssm_config e = c;
  e.batch = 0;
  EXPECT(rssm_decode_step(&e, &st, in, in, in, in, in, y, 0) == RSSM_OK);
  EXPECT(rssm_verify(&e, &st, 4, in, in, in, in, in, y, 0) == RSSM_OK);
  EXPECT(rssm_commit(&e, &st, iv, 4, 0) == RSSM_OK);
  EXPECT(rssm_flush(&e, &st, 16, 0) == RSSM_OK);
  EXPECT(rssm_stub_launches == 0);

  // --- valid arguments reach the launcher
  EXPECT(rssm_decode_step(&c, &st, in, in, in, in, in, y, 0) == RSSM_OK);
  EXPECT(rssm_verify(&c, &st, 4, in, in, in, in, in, y, 0) == RSSM_OK);
  EXPECT(rssm_stub_launches == 2);

  // --- every status and device bit has a message
  for (int code = -8; code <= 16; ++code) EXPECT(rssm_strerror(code) && strlen(rssm_strerror(code)) > 0);
  EXPECT(rssm_version() >= 100);

  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("ok\n");
  return 0;
}
