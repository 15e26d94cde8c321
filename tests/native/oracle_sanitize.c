/* Drives every oracle entry point at small sizes; built with AddressSanitizer and
 * UndefinedBehaviorSanitizer by tests/test_oracle_sanitized.py.  Every call gets
 * input and output buffers of exactly the documented size, so any access past them
 * is reported; a few results are cross-checked (round trips, definition vs fast
 * transform).  Exit status 0 on success. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/ntt_oracle.h"

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint64_t next64(void) { /* xorshift64*: test data only */
  state ^= state >> 12;
  state ^= state << 25;
  state ^= state >> 27;
  return state * 0x2545F4914F6CDD1Dull;
}
/* count residues laid out [..][limbs][n], limb t modulo q[t] */
static uint64_t *rnd(uint64_t count, uint64_t n, uint32_t limbs, const uint64_t *q) {
  uint64_t *x = malloc(count * sizeof(uint64_t));
  for (uint64_t i = 0; i < count; ++i) x[i] = next64() % q[(i / n) % limbs];
  return x;
}
static uint64_t *buf(uint64_t count) { return calloc(count, sizeof(uint64_t)); }
#define CHECK(c)                                                     \
  do {                                                               \
    if (!(c)) {                                                      \
      fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      return 1;                                                      \
    }                                                                \
  } while (0)

int main(void) {
  const uint64_t n = 16;
  uint64_t qp[12];
  CHECK(orc_find_primes(60, 2 * n, 12, qp) == 12);
  CHECK(orc_is_prime(qp[0]) && !orc_is_prime(qp[0] + 2));
  const uint64_t psi = orc_find_psi(qp[0], n);
  CHECK(psi && orc_pow_mod(psi, n, qp[0]) == qp[0] - 1);
  CHECK(orc_pow_mod(psi, 1, qp[0]) * 0 + (uint64_t)((unsigned __int128)orc_inv_mod(psi, qp[0]) * psi % qp[0]) == 1);

  /* single-limb transforms */
  uint64_t *a = rnd(n, n, 1, qp), *b = rnd(n, n, 1, qp), *c = buf(n), *d = buf(n);
  orc_ntt_definition(a, c, n, qp[0], psi);
  memcpy(d, a, n * 8);
  orc_ntt_forward(d, n, qp[0], psi);
  CHECK(memcmp(c, d, n * 8) == 0);
  orc_ntt_inverse(d, n, qp[0], psi);
  CHECK(memcmp(a, d, n * 8) == 0);
  orc_intt_definition(c, d, n, qp[0], psi);
  CHECK(memcmp(a, d, n * 8) == 0);
  orc_negacyclic_schoolbook(a, b, c, n, qp[0]);
  orc_automorph_coeff(a, d, n, qp[0], 5);
  orc_automorph_ntt(a, d, n, 5);
  free(a), free(b), free(c), free(d);

  /* batched drivers on [2][L][n] */
  const uint32_t L = 6;
  const uint64_t BL = 2 * L * n;
  uint64_t *x = rnd(BL, n, L, qp), *y = rnd(BL, n, L, qp), *z = buf(BL);
  memcpy(z, x, BL * 8);
  CHECK(orc_batch_ntt(z, 2, L, n, qp, 0, 2) == 0);
  CHECK(orc_batch_ntt(z, 2, L, n, qp, 1, 2) == 0);
  CHECK(memcmp(z, x, BL * 8) == 0);
  orc_batch_pointwise(z, x, y, 2, L, n, qp);
  uint64_t *t3 = buf(3 * L * n);
  orc_batch_tensor(t3, x, y, 1, L, n, qp); /* one ciphertext pair [2][L][n] -> [3][L][n] */
  free(t3);
  orc_batch_automorph(z, x, 25, 0, 2, L, n, qp);
  orc_batch_automorph(z, x, 25, 1, 2, L, n, qp);
  free(z);

  /* rescale: [2][L][n] -> [2][L-1][n] */
  uint64_t *r = buf(2 * (L - 1) * n);
  CHECK(orc_rescale(r, x, 0, 2, L, n, qp) == 0);
  CHECK(orc_rescale(r, x, 1, 2, L, n, qp) == 0);
  CHECK(orc_rescale(r, x, 2, 2, L, n, qp) == -1);
  free(r);

  /* CRT pieces */
  uint64_t words[16];
  CHECK(orc_crt_words(x, qp, 1, words, 16) >= 0);
  uint64_t col[12];
  for (int i = 0; i < 12; ++i) col[i] = qp[i] - 1;
  CHECK(orc_crt_words(col, qp, 12, words, 16) > 0);
  uint64_t *e4 = rnd(4 * n, n, 4, qp), *ext = buf(12 * n);
  orc_basis_extend(e4, 4, qp, ext, 12, qp, n);
  free(e4);
  uint64_t *acc = rnd(12 * n, n, 12, qp), *md = buf(8 * n);
  orc_moddown(acc, md, qp, 8, 4, n);
  free(acc), free(md), free(ext);

  /* modraise: [2][2][n] -> [2][12][n] */
  uint64_t *lo = rnd(2 * 2 * n, n, 2, qp), *up = buf(2 * 12 * n);
  CHECK(orc_modraise(up, lo, 2, 2, 12, n, qp) == 0);
  CHECK(orc_modraise(up, lo, 2, 2, 2, n, qp) == -1);
  free(lo), free(up);

  /* key-switch family: Q = 8 primes, P = 4, dnum = 2, batch 2 */
  const uint32_t nq = 8, np_ = 4, dnum = 2, nqp = 12;
  uint64_t *ct = rnd(2 * 2 * nq * n, n, nq, qp), *out = buf(2 * 2 * nq * n);
  uint64_t *ksk = rnd((uint64_t)dnum * 2 * nqp * n, n, nqp, qp);
  CHECK(orc_keyswitch(out, ct, ksk, 5, 2, n, qp, nq, np_, dnum, 2) == 0);
  CHECK(orc_keyswitch(out, ct, ksk, 4, 2, n, qp, nq, np_, dnum, 2) == -1); /* even g */
  uint64_t *dd = rnd(2 * 3 * nq * n, n, nq, qp);
  CHECK(orc_relinearize(out, dd, ksk, 2, n, qp, nq, np_, dnum, 2) == 0);
  free(dd);
  const uint64_t gs[2] = {5, 2 * n - 1};
  uint64_t *keys = rnd(2ull * dnum * 2 * nqp * n, n, nqp, qp), *hout = buf(2ull * 2 * 2 * nq * n);
  CHECK(orc_keyswitch_hoisted(hout, ct, keys, gs, 2, 2, n, qp, nq, np_, dnum, 2) == 0);
  free(keys), free(hout), free(ct), free(out), free(ksk), free(x), free(y);
  puts("oracle sanitized run ok");
  return 0;
}
