/* The C interface used from plain C99 (no C++, no Python): host-only entry
 * points, so it runs without a GPU.  Built and run by test_abi_host.py. */
#include <stdio.h>
#include <string.h>

#include "hsa.h"

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
  printf("c abi ok: n_active %d\n", (int)n);
  return 0;
}
