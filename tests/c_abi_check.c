/* The C interface used from plain C99 (no C++, no Python): host-only entry
 * points and the argument checks every entry point runs before it enqueues
 * anything, so it runs without a GPU (the device pointers below are aligned
 * placeholders that no rejected call dereferences).  Built and run by
 * test_abi_host.py, also against a host build with AddressSanitizer and
 * UndefinedBehaviorSanitizer. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "hsa.h"

#define DEV ((void *)(uintptr_t)0x10000) /* aligned placeholder, never dereferenced here */
#define EXPECT(call, code) \
  do {                     \
    if ((call) != (code)) { \
      printf("unexpected status from %s\n", #call); \
      return 1;            \
    }                      \
  } while (0)

/* Invalid calls of every entry point family: each returns its documented
 * status before anything is enqueued. */
static int check_rejections(void) {
  hsa_dims d;
  hsa_schedule s;
  hsa_block blk;
  hsa_model m;
  hsa_state st;
  int32_t counts[3] = {8190, 8190, 16380};
  int32_t bad_counts[3] = {8190, 8190, 16379};
  size_t ws = 0;
  memset(&d, 0, sizeof d);
  d.N = 256;
  d.C = 16;
  d.D = 128;
  d.H = 2;
  d.Dh = 64;
  d.F = 512;
  d.L = 1;
  d.dtype = HSA_F32;
  memset(&s, 0, sizeof s);
  s.T = 8;
  s.K = 2;
  s.budget[0] = 8;
  s.budget[1] = 4;
  s.count[0] = 128;
  s.count[1] = 128;
  memset(&blk, 0, sizeof blk);
  blk.w_qkv = blk.w_o = blk.w_1 = blk.w_2 = DEV;
  blk.k_cache = blk.v_cache = DEV;
  memset(&m, 0, sizeof m);
  m.dims = d;
  m.w_in = m.w_out = DEV;
  m.blocks = &blk;
  memset(&st, 0, sizeof st);
  st.x = st.v_hat = st.score = (float *)DEV;
  st.group = (uint8_t *)DEV;
  st.active_idx = st.pos = (int32_t *)DEV;
  st.workspace = DEV;
  st.workspace_bytes = 0; /* too small */
  EXPECT(hsa_workspace_size(NULL, &ws), HSA_ERR_ARG);
  EXPECT(hsa_step(&m, &s, &st, 0, 1.0f, 0.875f, 0, NULL, NULL), HSA_ERR_WORKSPACE);
  st.workspace_bytes = (size_t)1 << 40;
  EXPECT(hsa_step(&m, &s, &st, 8, 1.0f, 0.875f, 0, NULL, NULL), HSA_ERR_ARG);      /* iter >= T */
  EXPECT(hsa_step(&m, &s, &st, 0, 1.0f, 0.875f, 2, NULL, NULL), HSA_ERR_ARG);      /* regroup flag */
  s.budget[1] = 3;                                                                  /* 8 % 3 != 0 */
  EXPECT(hsa_step(&m, &s, &st, 0, 1.0f, 0.875f, 0, NULL, NULL), HSA_ERR_SCHEDULE);
  s.budget[1] = 4;
  s.count[1] = 127;                                                                 /* sum != N */
  EXPECT(hsa_step(&m, &s, &st, 0, 1.0f, 0.875f, 0, NULL, NULL), HSA_ERR_SCHEDULE);
  s.count[1] = 128;
  st.x = (float *)((uintptr_t)0x10002);                                             /* misaligned */
  EXPECT(hsa_step(&m, &s, &st, 0, 1.0f, 0.875f, 0, NULL, NULL), HSA_ERR_ALIGN);
  st.x = (float *)DEV;
  blk.w_o = NULL;
  EXPECT(hsa_step(&m, &s, &st, 0, 1.0f, 0.875f, 0, NULL, NULL), HSA_ERR_ARG);
  EXPECT(hsa_block_forward(&m, 0, (float *)DEV, (int32_t *)DEV, 4, NULL, 0, DEV, (size_t)1 << 40, NULL),
         HSA_ERR_ARG);
  blk.w_o = DEV;
  EXPECT(hsa_block_forward(&m, 1, (float *)DEV, (int32_t *)DEV, 4, NULL, 0, DEV, (size_t)1 << 40, NULL),
         HSA_ERR_ARG);                                                              /* layer >= L */
  EXPECT(hsa_block_forward(&m, 0, (float *)DEV, (int32_t *)DEV, 4, NULL, 1, DEV, (size_t)1 << 40, NULL),
         HSA_ERR_ARG);                                                              /* no guidance */
  m.dims.Dh = 96;
  EXPECT(hsa_step(&m, &s, &st, 0, 1.0f, 0.875f, 0, NULL, NULL), HSA_ERR_SHAPE);
  m.dims.Dh = 64;
  EXPECT(hsa_attn_active(DEV, DEV, DEV, DEV, 10, 100, 2, 96, 0.1f, HSA_BF16, NULL, 0, NULL),
         HSA_ERR_SHAPE);
  EXPECT(hsa_attn_active(DEV, DEV, DEV, DEV, 10, 100, 2, 64, -1.0f, HSA_BF16, NULL, 0, NULL),
         HSA_ERR_ARG);
  EXPECT(hsa_attn_active(DEV, DEV, DEV, DEV, 10, 100, 2, 64, 0.1f, (hsa_dtype)7, NULL, 0, NULL),
         HSA_ERR_DTYPE);
  EXPECT(hsa_attn_active_noalloc(DEV, DEV, DEV, DEV, 256, 75600, 200, 128, 0.088f, HSA_BF16, NULL),
         HSA_ERR_TOO_LARGE);
  EXPECT(hsa_attn_active_noalloc(NULL, DEV, DEV, DEV, 8, 64, 2, 128, 0.088f, HSA_BF16, NULL), HSA_ERR_ARG);
  EXPECT(hsa_euler((float *)DEV, (float *)DEV, (float *)DEV, (float *)DEV, (int32_t *)DEV, 100, 6, -0.1f,
                   1e-6f, 1, NULL),
         HSA_ERR_SHAPE);                                                            /* C % 4 */
  EXPECT(hsa_euler((float *)DEV, (float *)DEV, (float *)DEV, (float *)DEV, (int32_t *)DEV, 100, 16, -0.1f,
                   1e-6f, 2, NULL),
         HSA_ERR_ARG);
  EXPECT(hsa_select((float *)DEV, 32760, bad_counts, 3, (uint8_t *)DEV, NULL, 0, NULL), HSA_ERR_SCHEDULE);
  EXPECT(hsa_select((float *)DEV, 32760, counts, 9, (uint8_t *)DEV, NULL, 0, NULL), HSA_ERR_SHAPE);
  EXPECT(hsa_select_batch((float *)DEV, 0, 32760, counts, 3, (uint8_t *)DEV, NULL), HSA_ERR_SHAPE);
  EXPECT(hsa_select_batch((float *)DEV, 1 << 20, 1 << 20, counts, 3, (uint8_t *)DEV, NULL), HSA_ERR_SHAPE);
  EXPECT(hsa_active_set((uint8_t *)DEV, 256, &s, 8, (int32_t *)DEV, (int32_t *)DEV, (int32_t *)DEV, NULL),
         HSA_ERR_ARG);
  EXPECT(hsa_linear(DEV, DEV, DEV, 10, 64, 60, 0, HSA_BF16, NULL), HSA_ERR_SHAPE);  /* K % 64 */
  EXPECT(hsa_linear(DEV, DEV, DEV, 10, 64, 64, 2, HSA_BF16, NULL), HSA_ERR_ARG);    /* act */
  EXPECT(hsa_qkv_scatter(DEV, (int32_t *)DEV, 2, DEV, DEV, DEV, DEV, 4, 8, 64, HSA_BF16, NULL), HSA_ERR_ARG);
  EXPECT(hsa_qkv_scatter(DEV, (int32_t *)DEV, 0, DEV, DEV, DEV, DEV, 9, 8, 64, HSA_BF16, NULL),
         HSA_ERR_SHAPE);                                                            /* n_active > N */
  EXPECT(hsa_layernorm((float *)DEV, DEV, 4, 130, NULL, NULL, HSA_BF16, NULL), HSA_ERR_SHAPE);
  EXPECT(hsa_layernorm((float *)DEV, DEV, 4, 128, (float *)DEV, NULL, HSA_BF16, NULL), HSA_ERR_ARG);
  EXPECT(hsa_embed((float *)DEV, (int32_t *)DEV, DEV, (float *)DEV, -1, 16, 128, HSA_BF16, NULL), HSA_ERR_SHAPE);
  EXPECT(hsa_unembed((float *)DEV, DEV, (float *)DEV, 4, 130, 16, NULL, NULL, HSA_BF16, NULL), HSA_ERR_SHAPE);
  EXPECT(hsa_guidance((float *)DEV, (float *)DEV, 4, 16, 0.0f / 0.0f, NULL), HSA_ERR_ARG);
  return 0;
}

int main(void) {
  hsa_schedule s;
  hsa_dims d;
  int32_t n = -1;
  size_t ws = 0;
  if (hsa_abi_version() != HSA_ABI_VERSION) return 1;
  memset(&s, 0, sizeof s);
  s.T = 40;
  s.K = 3;
  s.budget[0] = 40;
  s.budget[1] = 20;
  s.budget[2] = 10;
  s.count[0] = 8190;
  s.count[1] = 8190;
  s.count[2] = 16380;
  /* |A_i| in closed form: all groups at i = 0, G_1 + G_2 at i = 2, G_1 at odd i */
  if (hsa_n_active(&s, 0, &n) != HSA_OK || n != 32760) return 2;
  if (hsa_n_active(&s, 2, &n) != HSA_OK || n != 16380) return 3;
  if (hsa_n_active(&s, 1, &n) != HSA_OK || n != 8190) return 4;
  if (hsa_n_active(&s, 40, &n) == HSA_OK) return 5; /* iteration out of range */
  memset(&d, 0, sizeof d);
  d.N = 32760;
  d.C = 16;
  d.D = 1536;
  d.H = 12;
  d.Dh = 128;
  d.F = 8960;
  d.L = 30;
  d.dtype = HSA_BF16;
  if (hsa_workspace_size(&d, &ws) != HSA_OK || ws == 0) return 6;
  d.Dh = 96; /* D != H * Dh */
  if (hsa_workspace_size(&d, &ws) != HSA_ERR_SHAPE) return 7;
  if (hsa_status_str(HSA_ERR_SHAPE) == NULL || strlen(hsa_status_str(HSA_ERR_SHAPE)) == 0) return 8;
  if (check_rejections() != 0) return 9;
  printf("c abi ok: n_active %d\n", (int)n);
  return 0;
}
