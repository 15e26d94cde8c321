/* Host-only paths of the library (no GPU): prime search, host plan creation with its
 * tables and validation, the query calls, and the argument checks of compute entry
 * points on host plans.  Built with AddressSanitizer + UBSan on the host side by
 * tests/test_host_sanitized.py.  Exit status 0 on success. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/negacyclic_ntt.h"

#define CHECK(c)                                                     \
  do {                                                               \
    if (!(c)) {                                                      \
      fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      return 1;                                                      \
    }                                                                \
  } while (0)

int main(void) {
  uint64_t q[8];
  const uint32_t sizes[] = {2, 16, 1024, 65536};
  const uint32_t bits[] = {20, 30, 60, 62};
  for (int si = 0; si < 4; ++si)
    for (int bi = 0; bi < 4; ++bi) {
      const uint32_t n = sizes[si];
      if (bits[bi] == 20 && n > 1024) continue;
      CHECK(ntt_find_primes(bits[bi], n, 3, q) == NTT_OK);
      ntt_plan *p = NULL;
      CHECK(ntt_plan_create(&p, n, q, 3, NULL, -1) == NTT_OK);
      uint64_t *t = malloc((size_t)n * 4 * sizeof(uint64_t)), psi = 0;
      CHECK(ntt_plan_get_tables(p, 2, &psi, t, t + n, t + 2 * n, t + 3 * n) == NTT_OK);
      CHECK(psi != 0 && t[0] == 1 && t[2 * n] == 1);
      CHECK(ntt_plan_get_tables(p, 3, NULL, NULL, NULL, NULL, NULL) == NTT_EINVAL);
      uint32_t nn = 0, np = 0;
      int dev = 0;
      CHECK(ntt_plan_info(p, &nn, &np, &dev) == NTT_OK && nn == n && np == 3 && dev == -1);
      uint64_t qq = 0;
      CHECK(ntt_plan_prime(p, 1, &qq) == NTT_OK && qq == q[1]);
      void *fake = (void *)0x1000;
      CHECK(ntt_forward(p, fake, 1, 0, 3, NULL) == NTT_EDEVICE);
      CHECK(rescale(p, fake, fake, 0, 1, 0, 3, NULL) == NTT_EDEVICE);
      ntt_ks_plan *ks = NULL;
      CHECK(keyswitch_plan_create(&ks, p, 2, 1, 1) == NTT_EDEVICE);
      ntt_mr_plan *mr = NULL;
      CHECK(modraise_plan_create(&mr, p, 1, 2) == NTT_EDEVICE);
      free(t);
      ntt_plan_destroy(p);
    }
  /* validation failures */
  ntt_plan *p = NULL;
  CHECK(ntt_find_primes(2, 4, 1, q) != NTT_OK);
  CHECK(ntt_find_primes(30, 3, 1, q) != NTT_OK);
  CHECK(ntt_find_primes(30, 1024, 2, q) == NTT_OK);
  CHECK(ntt_plan_create(&p, 1000, q, 2, NULL, -1) == NTT_EINVAL);
  uint64_t dup[2] = {q[0], q[0]};
  CHECK(ntt_plan_create(&p, 1024, dup, 2, NULL, -1) == NTT_EINVAL);
  uint64_t comp[1] = {q[0] + 2 * 1024 * 2};
  (void)ntt_plan_create(&p, 1024, comp, 1, NULL, -1); /* prime or not: no crash */
  if (p) ntt_plan_destroy(p), p = NULL;
  uint64_t badpsi[2] = {3, 3};
  CHECK(ntt_plan_create(&p, 1024, q, 2, badpsi, -1) == NTT_EINVAL);
  CHECK(ntt_plan_create(NULL, 1024, q, 2, NULL, -1) == NTT_EINVAL);
  CHECK(strlen(ntt_status_string(NTT_EOVERLAP)) > 0);
  ntt_plan_destroy(NULL);
  keyswitch_plan_destroy(NULL);
  modraise_plan_destroy(NULL);
  puts("host sanitized run ok");
  return 0;
}
