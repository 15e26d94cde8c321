/*
 * ntt_oracle.c -- plain C reference for the negacyclic NTT library.
 *
 * TEST INFRASTRUCTURE ONLY (see ntt_oracle.h): slow, obviously correct, shares
 * nothing with the GPU library.  Every modular product is a 128-bit product
 * reduced with the `%` operator; multi-prime values are built as explicit
 * multi-word integers.
 */
#include "ntt_oracle.h"

#include <pthread.h>
#include <stdlib.h>
#include <string.h>

typedef unsigned __int128 u128;

/* ---- scalar modular arithmetic (a, b canonical unless noted) ------------- */

static uint64_t mulm(uint64_t a, uint64_t b, uint64_t q) { return (uint64_t)(((u128)a * b) % q); }
static uint64_t addm(uint64_t a, uint64_t b, uint64_t q) { return (uint64_t)(((u128)a + b) % q); }
static uint64_t subm(uint64_t a, uint64_t b, uint64_t q) { return (uint64_t)(((u128)a + q - b) % q); }
static uint64_t negm(uint64_t a, uint64_t q) { return a == 0 ? 0 : q - a; }

uint64_t orc_pow_mod(uint64_t b, uint64_t e, uint64_t q) {
  uint64_t r = 1 % q;
  b %= q;
  while (e) {
    if (e & 1) r = mulm(r, b, q);
    b = mulm(b, b, q);
    e >>= 1;
  }
  return r;
}

/* q prime: a^(q-2) (Fermat). */
uint64_t orc_inv_mod(uint64_t a, uint64_t q) { return orc_pow_mod(a % q, q - 2, q); }

static unsigned log2u(uint64_t n) {
  unsigned m = 0;
  while ((1ull << m) < n) ++m;
  return m;
}

static uint64_t bitrev(uint64_t x, unsigned bits) {
  uint64_t r = 0;
  for (unsigned i = 0; i < bits; ++i) r |= ((x >> i) & 1ull) << (bits - 1 - i);
  return r;
}

/* ---- primes and roots ----------------------------------------------------- */

int orc_is_prime(uint64_t n) {
  static const uint64_t bases[12] = {2, 3, 5, 7, 11, 13, 17, 19, 23, 29, 31, 37};
  if (n < 2) return 0;
  for (int i = 0; i < 12; ++i)
    if (n % bases[i] == 0) return n == bases[i];
  uint64_t d = n - 1;
  int s = 0;
  while ((d & 1) == 0) {
    d >>= 1;
    ++s;
  }
  for (int i = 0; i < 12; ++i) {
    uint64_t x = orc_pow_mod(bases[i], d, n);
    if (x == 1 || x == n - 1) continue;
    int witness = 1;
    for (int r = 1; r < s; ++r) {
      x = mulm(x, x, n);
      if (x == n - 1) {
        witness = 0;
        break;
      }
    }
    if (witness) return 0;
  }
  return 1;
}

uint32_t orc_find_primes(uint32_t bits, uint64_t two_n, uint32_t count, uint64_t *out) {
  if (bits < 2 || bits > 63 || two_n == 0) return 0;
  uint64_t top = (1ull << bits) - 2; /* candidates are <= 2^bits - 1 */
  uint64_t c = (top / two_n) * two_n + 1;
  uint32_t found = 0;
  while (found < count && c > two_n) {
    if (orc_is_prime(c)) out[found++] = c;
    c -= two_n;
  }
  return found;
}

uint64_t orc_find_psi(uint64_t q, uint64_t n) {
  if (q < 3 || n == 0 || (q - 1) % (2 * n) != 0) return 0;
  /* Find one element of order exactly 2n: r = x^((q-1)/2n) with r^n == -1. */
  uint64_t r = 0;
  for (uint64_t x = 2; x < q; ++x) {
    uint64_t c = orc_pow_mod(x, (q - 1) / (2 * n), q);
    if (orc_pow_mod(c, n, q) == q - 1) {
      r = c;
      break;
    }
  }
  if (!r) return 0;
  /* Every x with x^n == -1 is an odd power of r; take the smallest. */
  uint64_t best = r, r2 = mulm(r, r, q), p = r;
  for (uint64_t k = 1; k < n; ++k) {
    p = mulm(p, r2, q);
    if (p < best) best = p;
  }
  return best;
}

/* ---- transforms ----------------------------------------------------------- */

void orc_ntt_definition(const uint64_t *a, uint64_t *out, uint64_t n, uint64_t q, uint64_t psi) {
  unsigned m = log2u(n);
  uint64_t two_n = 2 * n;
  uint64_t *pw = (uint64_t *)malloc(two_n * sizeof(uint64_t));
  pw[0] = 1 % q;
  for (uint64_t e = 1; e < two_n; ++e) pw[e] = mulm(pw[e - 1], psi, q);
  for (uint64_t k = 0; k < n; ++k) {
    uint64_t ek = 2 * bitrev(k, m) + 1, acc = 0;
    for (uint64_t i = 0; i < n; ++i) acc = addm(acc, mulm(a[i], pw[(uint64_t)(((u128)ek * i) % two_n)], q), q);
    out[k] = acc;
  }
  free(pw);
}

void orc_intt_definition(const uint64_t *ahat, uint64_t *out, uint64_t n, uint64_t q, uint64_t psi) {
  unsigned m = log2u(n);
  uint64_t two_n = 2 * n, psi_inv = orc_inv_mod(psi, q), n_inv = orc_inv_mod(n % q, q);
  uint64_t *pw = (uint64_t *)malloc(two_n * sizeof(uint64_t));
  pw[0] = 1 % q;
  for (uint64_t e = 1; e < two_n; ++e) pw[e] = mulm(pw[e - 1], psi_inv, q);
  for (uint64_t i = 0; i < n; ++i) {
    uint64_t acc = 0;
    for (uint64_t k = 0; k < n; ++k) {
      uint64_t ek = 2 * bitrev(k, m) + 1;
      acc = addm(acc, mulm(ahat[k], pw[(uint64_t)(((u128)ek * i) % two_n)], q), q);
    }
    out[i] = mulm(acc, n_inv, q);
  }
  free(pw);
}

/* table[k] = w^brv(k) for k < n. */
static uint64_t *brv_power_table(uint64_t w, uint64_t n, uint64_t q) {
  unsigned m = log2u(n);
  uint64_t *pw = (uint64_t *)malloc(n * sizeof(uint64_t));
  uint64_t *tab = (uint64_t *)malloc(n * sizeof(uint64_t));
  pw[0] = 1 % q;
  for (uint64_t e = 1; e < n; ++e) pw[e] = mulm(pw[e - 1], w, q);
  for (uint64_t k = 0; k < n; ++k) tab[k] = pw[bitrev(k, m)];
  free(pw);
  return tab;
}

void orc_ntt_forward(uint64_t *a, uint64_t n, uint64_t q, uint64_t psi) {
  uint64_t *tab = brv_power_table(psi, n, q);
  uint64_t t = n;
  for (uint64_t m = 1; m < n; m <<= 1) {
    t >>= 1;
    for (uint64_t i = 0; i < m; ++i) {
      uint64_t j1 = 2 * i * t, s = tab[m + i];
      for (uint64_t j = j1; j < j1 + t; ++j) {
        uint64_t u = a[j], v = mulm(a[j + t], s, q);
        a[j] = addm(u, v, q);
        a[j + t] = subm(u, v, q);
      }
    }
  }
  free(tab);
}

void orc_ntt_inverse(uint64_t *a, uint64_t n, uint64_t q, uint64_t psi) {
  uint64_t *tab = brv_power_table(orc_inv_mod(psi, q), n, q);
  uint64_t t = 1;
  for (uint64_t m = n; m > 1; m >>= 1) {
    uint64_t h = m >> 1, j1 = 0;
    for (uint64_t i = 0; i < h; ++i) {
      uint64_t s = tab[h + i];
      for (uint64_t j = j1; j < j1 + t; ++j) {
        uint64_t u = a[j], v = a[j + t];
        a[j] = addm(u, v, q);
        a[j + t] = mulm(subm(u, v, q), s, q);
      }
      j1 += 2 * t;
    }
    t <<= 1;
  }
  uint64_t n_inv = orc_inv_mod(n % q, q);
  for (uint64_t j = 0; j < n; ++j) a[j] = mulm(a[j], n_inv, q);
  free(tab);
}

void orc_negacyclic_schoolbook(const uint64_t *a, const uint64_t *b, uint64_t *c, uint64_t n, uint64_t q) {
  uint64_t *acc = (uint64_t *)calloc(n, sizeof(uint64_t));
  for (uint64_t i = 0; i < n; ++i)
    for (uint64_t j = 0; j < n; ++j) {
      uint64_t p = mulm(a[i], b[j], q);
      if (i + j < n)
        acc[i + j] = addm(acc[i + j], p, q);
      else
        acc[i + j - n] = subm(acc[i + j - n], p, q); /* X^n = -1 */
    }
  memcpy(c, acc, n * sizeof(uint64_t));
  free(acc);
}

void orc_automorph_coeff(const uint64_t *in, uint64_t *out, uint64_t n, uint64_t q, uint64_t g) {
  uint64_t two_n = 2 * n;
  for (uint64_t i = 0; i < n; ++i) {
    uint64_t e = (uint64_t)(((u128)i * g) % two_n);
    if (e < n)
      out[e] = in[i];
    else
      out[e - n] = negm(in[i], q);
  }
}

void orc_automorph_ntt(const uint64_t *in, uint64_t *out, uint64_t n, uint64_t g) {
  unsigned m = log2u(n);
  uint64_t two_n = 2 * n;
  for (uint64_t k = 0; k < n; ++k) {
    uint64_t e = (uint64_t)(((u128)(2 * bitrev(k, m) + 1) * g) % two_n); /* odd */
    out[k] = in[bitrev((e - 1) / 2, m)];
  }
}

/* ---- a tiny parallel-for -------------------------------------------------- */

typedef void (*work_fn)(void *ctx, uint64_t unit);
typedef struct {
  work_fn fn;
  void *ctx;
  uint64_t count;
  uint64_t next; /* atomic */
} pool_t;

static void *pool_worker(void *arg) {
  pool_t *p = (pool_t *)arg;
  for (;;) {
    uint64_t u = __atomic_fetch_add(&p->next, 1, __ATOMIC_RELAXED);
    if (u >= p->count) break;
    p->fn(p->ctx, u);
  }
  return NULL;
}

static void parallel_for(uint64_t count, work_fn fn, void *ctx, int threads) {
  pool_t p = {fn, ctx, count, 0};
  if (threads <= 1 || count <= 1) {
    pool_worker(&p);
    return;
  }
  if ((uint64_t)threads > count) threads = (int)count;
  pthread_t *tid = (pthread_t *)malloc((size_t)threads * sizeof(pthread_t));
  int started = 0;
  for (int t = 1; t < threads; ++t) {
    pthread_t th;
    if (pthread_create(&th, NULL, pool_worker, &p) == 0) tid[started++] = th;
  }
  /* The calling thread works too; then join every thread that started. */
  pool_worker(&p);
  for (int t = 0; t < started; ++t) pthread_join(tid[t], NULL);
  free(tid);
}

/* ---- batched drivers ------------------------------------------------------ */

typedef struct {
  uint64_t *data;
  uint32_t limbs;
  uint64_t n;
  const uint64_t *primes;
  const uint64_t *psis;
  int inverse;
} batch_ntt_ctx;

static void batch_ntt_unit(void *vctx, uint64_t u) {
  batch_ntt_ctx *c = (batch_ntt_ctx *)vctx;
  uint32_t l = (uint32_t)(u % c->limbs);
  uint64_t *row = c->data + u * c->n;
  if (c->inverse)
    orc_ntt_inverse(row, c->n, c->primes[l], c->psis[l]);
  else
    orc_ntt_forward(row, c->n, c->primes[l], c->psis[l]);
}

int orc_batch_ntt(uint64_t *data, uint64_t batch, uint32_t limbs, uint64_t n, const uint64_t *primes,
                  int inverse, int threads) {
  uint64_t *psis = (uint64_t *)malloc((limbs ? limbs : 1) * sizeof(uint64_t));
  for (uint32_t l = 0; l < limbs; ++l) {
    psis[l] = orc_find_psi(primes[l], n);
    if (!psis[l]) {
      free(psis);
      return -1;
    }
  }
  batch_ntt_ctx ctx = {data, limbs, n, primes, psis, inverse};
  parallel_for(batch * limbs, batch_ntt_unit, &ctx, threads);
  free(psis);
  return 0;
}

void orc_batch_pointwise(uint64_t *out, const uint64_t *a, const uint64_t *b, uint64_t batch, uint32_t limbs,
                         uint64_t n, const uint64_t *primes) {
  for (uint64_t bi = 0; bi < batch; ++bi)
    for (uint32_t l = 0; l < limbs; ++l) {
      uint64_t off = (bi * limbs + l) * n, q = primes[l];
      for (uint64_t e = 0; e < n; ++e) out[off + e] = mulm(a[off + e], b[off + e], q);
    }
}

void orc_batch_tensor(uint64_t *out, const uint64_t *a, const uint64_t *b, uint64_t batch, uint32_t limbs,
                      uint64_t n, const uint64_t *primes) {
  uint64_t plane = (uint64_t)limbs * n;
  for (uint64_t bi = 0; bi < batch; ++bi) {
    const uint64_t *a0 = a + bi * 2 * plane, *a1 = a0 + plane;
    const uint64_t *b0 = b + bi * 2 * plane, *b1 = b0 + plane;
    uint64_t *d0 = out + bi * 3 * plane, *d1 = d0 + plane, *d2 = d1 + plane;
    for (uint32_t l = 0; l < limbs; ++l) {
      uint64_t q = primes[l];
      for (uint64_t e = 0; e < n; ++e) {
        uint64_t i = (uint64_t)l * n + e;
        d0[i] = mulm(a0[i], b0[i], q);
        d1[i] = addm(mulm(a0[i], b1[i], q), mulm(a1[i], b0[i], q), q);
        d2[i] = mulm(a1[i], b1[i], q);
      }
    }
  }
}

void orc_batch_automorph(uint64_t *out, const uint64_t *in, uint64_t g, int domain, uint64_t batch,
                         uint32_t limbs, uint64_t n, const uint64_t *primes) {
  for (uint64_t bi = 0; bi < batch; ++bi)
    for (uint32_t l = 0; l < limbs; ++l) {
      uint64_t off = (bi * limbs + l) * n;
      if (domain == 0)
        orc_automorph_coeff(in + off, out + off, n, primes[l], g);
      else
        orc_automorph_ntt(in + off, out + off, n, g);
    }
}

/* ---- multi-word integers (little-endian 64-bit words) --------------------- */

#define ORC_MAXW 72

typedef struct {
  uint32_t len; /* significant words */
  uint64_t w[ORC_MAXW];
} big_t;

static void big_set_u64(big_t *x, uint64_t v) {
  memset(x, 0, sizeof(*x));
  x->w[0] = v;
  x->len = v ? 1 : 0;
}

static void big_norm(big_t *x) {
  while (x->len && x->w[x->len - 1] == 0) --x->len;
}

/* x *= m; returns -1 on overflow of the fixed capacity. */
static int big_mul_u64(big_t *x, uint64_t m) {
  u128 carry = 0;
  for (uint32_t i = 0; i < x->len; ++i) {
    u128 t = (u128)x->w[i] * m + carry;
    x->w[i] = (uint64_t)t;
    carry = t >> 64;
  }
  if (carry) {
    if (x->len >= ORC_MAXW) return -1;
    x->w[x->len++] = (uint64_t)carry;
  }
  big_norm(x);
  return 0;
}

/* r = a * m (a big, m u64) */
static int big_mul_small(big_t *r, const big_t *a, uint64_t m) {
  *r = *a;
  return big_mul_u64(r, m);
}

/* x += y */
static int big_add(big_t *x, const big_t *y) {
  uint32_t len = x->len > y->len ? x->len : y->len;
  u128 carry = 0;
  for (uint32_t i = 0; i < len; ++i) {
    u128 t = (u128)x->w[i] + y->w[i] + carry;
    x->w[i] = (uint64_t)t;
    carry = t >> 64;
  }
  x->len = len;
  if (carry) {
    if (len >= ORC_MAXW) return -1;
    x->w[x->len++] = 1;
  }
  return 0;
}

static int big_cmp(const big_t *x, const big_t *y) {
  if (x->len != y->len) return x->len < y->len ? -1 : 1;
  for (uint32_t i = x->len; i-- > 0;)
    if (x->w[i] != y->w[i]) return x->w[i] < y->w[i] ? -1 : 1;
  return 0;
}

/* x -= y, requires x >= y */
static void big_sub(big_t *x, const big_t *y) {
  uint64_t borrow = 0;
  for (uint32_t i = 0; i < x->len; ++i) {
    uint64_t yi = i < y->len ? y->w[i] : 0;
    u128 t = (u128)x->w[i] - yi - borrow;
    x->w[i] = (uint64_t)t;
    borrow = (uint64_t)(t >> 127); /* 1 if it wrapped */
  }
  big_norm(x);
}

static uint64_t big_mod_u64(const big_t *x, uint64_t m) {
  u128 r = 0;
  for (uint32_t i = x->len; i-- > 0;) r = ((r << 64) | x->w[i]) % m;
  return (uint64_t)r;
}

/* exact division by a single word: q = x / m (m must divide x) */
static void big_div_u64(big_t *quo, const big_t *x, uint64_t m) {
  memset(quo, 0, sizeof(*quo));
  u128 r = 0;
  for (uint32_t i = x->len; i-- > 0;) {
    u128 cur = (r << 64) | x->w[i];
    quo->w[i] = (uint64_t)(cur / m);
    r = cur % m;
  }
  quo->len = x->len;
  big_norm(quo);
}

/* Precomputed CRT basis: M = prod m_t, Mt = M / m_t, ct = (Mt mod m_t)^-1 mod m_t. */
typedef struct {
  uint32_t k;
  const uint64_t *m;
  big_t M;
  big_t *Mt;
  uint64_t *ct;
} crt_basis;

static int crt_basis_init(crt_basis *b, const uint64_t *m, uint32_t k) {
  b->k = k;
  b->m = m;
  b->Mt = (big_t *)malloc((k ? k : 1) * sizeof(big_t));
  b->ct = (uint64_t *)malloc((k ? k : 1) * sizeof(uint64_t));
  big_set_u64(&b->M, 1);
  for (uint32_t t = 0; t < k; ++t)
    if (big_mul_u64(&b->M, m[t])) return -1;
  for (uint32_t t = 0; t < k; ++t) {
    big_div_u64(&b->Mt[t], &b->M, m[t]);
    b->ct[t] = orc_inv_mod(big_mod_u64(&b->Mt[t], m[t]), m[t]);
  }
  return 0;
}

static void crt_basis_free(crt_basis *b) {
  free(b->Mt);
  free(b->ct);
}

/* X = sum_t (x_t * ct mod m_t) * Mt, reduced into [0, M). */
static int crt_value(const crt_basis *b, const uint64_t *x, uint64_t stride, big_t *X) {
  big_set_u64(X, 0);
  for (uint32_t t = 0; t < b->k; ++t) {
    big_t term;
    if (big_mul_small(&term, &b->Mt[t], mulm(x[t * stride] % b->m[t], b->ct[t], b->m[t]))) return -1;
    if (big_add(X, &term)) return -1;
  }
  while (big_cmp(X, &b->M) >= 0) big_sub(X, &b->M);
  return 0;
}

int orc_crt_words(const uint64_t *x, const uint64_t *m, uint32_t k, uint64_t *out, uint32_t words) {
  crt_basis b;
  big_t X;
  int rc = -1;
  if (crt_basis_init(&b, m, k) == 0 && crt_value(&b, x, 1, &X) == 0 && X.len <= words) {
    memset(out, 0, words * sizeof(uint64_t));
    memcpy(out, X.w, X.len * sizeof(uint64_t));
    rc = (int)X.len;
  }
  crt_basis_free(&b);
  return rc;
}

/* ---- basis extension and ModDown ------------------------------------------ */

typedef struct {
  const uint64_t *x;
  const crt_basis *b;
  uint64_t *out;
  uint32_t m;
  const uint64_t *dst;
  uint64_t n;
} extend_ctx;

static void extend_unit(void *vctx, uint64_t e) {
  extend_ctx *c = (extend_ctx *)vctx;
  big_t D;
  crt_value(c->b, c->x + e, c->n, &D);
  for (uint32_t t = 0; t < c->m; ++t) c->out[(uint64_t)t * c->n + e] = big_mod_u64(&D, c->dst[t]);
}

static void basis_extend_threads(const uint64_t *x, uint32_t k, const uint64_t *src, uint64_t *out, uint32_t m,
                                 const uint64_t *dst, uint64_t n, int threads) {
  crt_basis b;
  crt_basis_init(&b, src, k);
  extend_ctx ctx = {x, &b, out, m, dst, n};
  parallel_for(n, extend_unit, &ctx, threads);
  crt_basis_free(&b);
}

void orc_basis_extend(const uint64_t *x, uint32_t k, const uint64_t *src, uint64_t *out, uint32_t m,
                      const uint64_t *dst, uint64_t n) {
  basis_extend_threads(x, k, src, out, m, dst, n, 1);
}

typedef struct {
  const uint64_t *acc;
  uint64_t *out;
  const uint64_t *qp;
  uint32_t nq;
  const crt_basis *pb;
  const uint64_t *p_inv; /* P^-1 mod q_l */
  uint64_t n;
} moddown_ctx;

static void moddown_unit(void *vctx, uint64_t e) {
  moddown_ctx *c = (moddown_ctx *)vctx;
  /* r = X mod P from the P residues; then floor(X/P) = (X - r) / P and, modulo
   * q_l, X == acc_l, so floor(X/P) mod q_l = (acc_l - r) * P^-1 mod q_l. */
  big_t r;
  crt_value(c->pb, c->acc + (uint64_t)c->nq * c->n + e, c->n, &r);
  for (uint32_t l = 0; l < c->nq; ++l) {
    uint64_t q = c->qp[l];
    uint64_t diff = subm(c->acc[(uint64_t)l * c->n + e], big_mod_u64(&r, q), q);
    c->out[(uint64_t)l * c->n + e] = mulm(diff, c->p_inv[l], q);
  }
}

static void moddown_threads(const uint64_t *acc, uint64_t *out, const uint64_t *qp, uint32_t nq, uint32_t np,
                            uint64_t n, int threads) {
  crt_basis pb;
  crt_basis_init(&pb, qp + nq, np);
  uint64_t *p_inv = (uint64_t *)malloc((nq ? nq : 1) * sizeof(uint64_t));
  for (uint32_t l = 0; l < nq; ++l) p_inv[l] = orc_inv_mod(big_mod_u64(&pb.M, qp[l]), qp[l]);
  moddown_ctx ctx = {acc, out, qp, nq, &pb, p_inv, n};
  parallel_for(n, moddown_unit, &ctx, threads);
  free(p_inv);
  crt_basis_free(&pb);
}

void orc_moddown(const uint64_t *acc, uint64_t *out, const uint64_t *qp, uint32_t nq, uint32_t np, uint64_t n) {
  moddown_threads(acc, out, qp, nq, np, n, 1);
}

/* ---- rotation key-switch --------------------------------------------------- */

int orc_keyswitch(uint64_t *out, const uint64_t *ct, const uint64_t *ksk, uint64_t g, uint64_t batch,
                  uint64_t n, const uint64_t *qp, uint32_t nq, uint32_t np, uint32_t dnum, int threads) {
  if (dnum == 0 || nq == 0 || nq % dnum != 0 || (g & 1) == 0) return -1;
  uint32_t nqp = nq + np, alpha = nq / dnum;
  uint64_t plane = (uint64_t)nq * n;
  uint64_t *rot = (uint64_t *)malloc(2 * plane * sizeof(uint64_t));
  uint64_t *ext = (uint64_t *)malloc((uint64_t)dnum * nqp * n * sizeof(uint64_t));
  uint64_t *acc = (uint64_t *)malloc(2 * (uint64_t)nqp * n * sizeof(uint64_t));
  uint64_t *md = (uint64_t *)malloc(plane * sizeof(uint64_t));
  int rc = 0;
  for (uint64_t bi = 0; bi < batch && rc == 0; ++bi) {
    const uint64_t *c = ct + bi * 2 * plane;
    uint64_t *o = out + bi * 2 * plane;
    /* 1. sigma_g on both components */
    for (int comp = 0; comp < 2; ++comp)
      for (uint32_t l = 0; l < nq; ++l)
        orc_automorph_coeff(c + comp * plane + (uint64_t)l * n, rot + comp * plane + (uint64_t)l * n, n, qp[l], g);
    /* 2-3. decompose c1' into dnum digits and extend each onto Q u P */
    for (uint32_t j = 0; j < dnum; ++j)
      basis_extend_threads(rot + plane + (uint64_t)j * alpha * n, alpha, qp + (uint64_t)j * alpha,
                           ext + (uint64_t)j * nqp * n, nqp, qp, n, threads);
    /* 4. NTT of every extended digit: limb t of each digit uses qp[t] */
    if (orc_batch_ntt(ext, dnum, nqp, n, qp, 0, threads)) rc = -1;
    /* 5. inner product with the key, per limb */
    for (int comp = 0; comp < 2; ++comp)
      for (uint32_t t = 0; t < nqp; ++t) {
        uint64_t q = qp[t];
        uint64_t *a = acc + ((uint64_t)comp * nqp + t) * n;
        for (uint64_t e = 0; e < n; ++e) {
          uint64_t s = 0;
          for (uint32_t j = 0; j < dnum; ++j)
            s = addm(s, mulm(ext[((uint64_t)j * nqp + t) * n + e], ksk[(((uint64_t)j * 2 + comp) * nqp + t) * n + e], q), q);
          a[e] = s;
        }
      }
    /* 6. back to the coefficient domain */
    if (orc_batch_ntt(acc, 2, nqp, n, qp, 1, threads)) rc = -1;
    /* 7-8. ModDown each component, add sigma_g(c0) */
    for (int comp = 0; comp < 2; ++comp) {
      moddown_threads(acc + (uint64_t)comp * nqp * n, md, qp, nq, np, n, threads);
      for (uint32_t l = 0; l < nq; ++l)
        for (uint64_t e = 0; e < n; ++e) {
          uint64_t i = (uint64_t)l * n + e;
          o[comp * plane + i] = comp == 0 ? addm(rot[i], md[i], qp[l]) : md[i];
        }
    }
  }
  free(rot);
  free(ext);
  free(acc);
  free(md);
  return rc;
}

/* ---- hoisted rotations ------------------------------------------------------ */

int orc_keyswitch_hoisted(uint64_t *out, const uint64_t *ct, const uint64_t *ksk, const uint64_t *gs, uint32_t R,
                          uint64_t batch, uint64_t n, const uint64_t *qp, uint32_t nq, uint32_t np, uint32_t dnum,
                          int threads) {
  if (dnum == 0 || nq == 0 || nq % dnum != 0 || R == 0) return -1;
  for (uint32_t r = 0; r < R; ++r)
    if ((gs[r] & 1) == 0) return -1;
  uint32_t nqp = nq + np, alpha = nq / dnum;
  uint64_t plane = (uint64_t)nq * n, qplane = (uint64_t)nqp * n;
  uint64_t *ext = (uint64_t *)malloc((uint64_t)dnum * qplane * sizeof(uint64_t));
  uint64_t *perm = (uint64_t *)malloc((uint64_t)dnum * qplane * sizeof(uint64_t));
  uint64_t *acc = (uint64_t *)malloc(2 * qplane * sizeof(uint64_t));
  uint64_t *md = (uint64_t *)malloc(plane * sizeof(uint64_t));
  uint64_t *c0r = (uint64_t *)malloc(plane * sizeof(uint64_t));
  int rc = 0;
  for (uint64_t bi = 0; bi < batch && rc == 0; ++bi) {
    const uint64_t *c0 = ct + bi * 2 * plane, *c1 = c0 + plane;
    /* decompose c1 (no automorphism) and extend every digit onto Q u P, then NTT */
    for (uint32_t j = 0; j < dnum; ++j)
      basis_extend_threads(c1 + (uint64_t)j * alpha * n, alpha, qp + (uint64_t)j * alpha, ext + (uint64_t)j * qplane,
                           nqp, qp, n, threads);
    if (orc_batch_ntt(ext, dnum, nqp, n, qp, 0, threads)) rc = -1;
    for (uint32_t r = 0; r < R && rc == 0; ++r) {
      const uint64_t g = gs[r];
      const uint64_t *k = ksk + (uint64_t)r * dnum * 2 * qplane;
      uint64_t *o = out + (r * batch + bi) * 2 * plane;
      /* the automorphism of every extended digit, in the NTT domain */
      for (uint64_t row = 0; row < (uint64_t)dnum * nqp; ++row) orc_automorph_ntt(ext + row * n, perm + row * n, n, g);
      for (int comp = 0; comp < 2; ++comp)
        for (uint32_t t = 0; t < nqp; ++t) {
          uint64_t q = qp[t];
          uint64_t *a = acc + ((uint64_t)comp * nqp + t) * n;
          for (uint64_t e = 0; e < n; ++e) {
            uint64_t s = 0;
            for (uint32_t j = 0; j < dnum; ++j)
              s = addm(s, mulm(perm[((uint64_t)j * nqp + t) * n + e], k[(((uint64_t)j * 2 + comp) * nqp + t) * n + e], q),
                       q);
            a[e] = s;
          }
        }
      if (orc_batch_ntt(acc, 2, nqp, n, qp, 1, threads)) rc = -1;
      for (uint32_t l = 0; l < nq; ++l) orc_automorph_coeff(c0 + (uint64_t)l * n, c0r + (uint64_t)l * n, n, qp[l], g);
      for (int comp = 0; comp < 2; ++comp) {
        moddown_threads(acc + (uint64_t)comp * qplane, md, qp, nq, np, n, threads);
        for (uint32_t l = 0; l < nq; ++l)
          for (uint64_t e = 0; e < n; ++e) {
            uint64_t i = (uint64_t)l * n + e;
            o[comp * plane + i] = comp == 0 ? addm(c0r[i], md[i], qp[l]) : md[i];
          }
      }
    }
  }
  free(ext);
  free(perm);
  free(acc);
  free(md);
  free(c0r);
  return rc;
}

/* ---- relinearisation -------------------------------------------------------- */

int orc_relinearize(uint64_t *out, const uint64_t *d, const uint64_t *rlk, uint64_t batch, uint64_t n,
                    const uint64_t *qp, uint32_t nq, uint32_t np, uint32_t dnum, int threads) {
  if (dnum == 0 || nq == 0 || nq % dnum != 0) return -1;
  uint64_t plane = (uint64_t)nq * n;
  uint64_t *ct = (uint64_t *)malloc(2 * plane * sizeof(uint64_t));
  int rc = 0;
  for (uint64_t bi = 0; bi < batch && rc == 0; ++bi) {
    const uint64_t *d0 = d + bi * 3 * plane, *d1 = d0 + plane, *d2 = d1 + plane;
    uint64_t *o = out + bi * 2 * plane;
    /* switch (d0, d2) with g = 1: gives (d0 + ModDown(acc_0), ModDown(acc_1)) */
    memcpy(ct, d0, plane * sizeof(uint64_t));
    memcpy(ct + plane, d2, plane * sizeof(uint64_t));
    rc = orc_keyswitch(o, ct, rlk, 1, 1, n, qp, nq, np, dnum, threads);
    for (uint32_t l = 0; l < nq && rc == 0; ++l)
      for (uint64_t e = 0; e < n; ++e) {
        uint64_t i = (uint64_t)l * n + e;
        o[plane + i] = addm(o[plane + i], d1[i], qp[l]);
      }
  }
  free(ct);
  return rc;
}

/* ---- rescale ---------------------------------------------------------------- */

int orc_rescale(uint64_t *out, const uint64_t *in, int mode, uint64_t batch, uint32_t limbs, uint64_t n,
                const uint64_t *primes) {
  if (limbs < 2 || (mode != 0 && mode != 1)) return -1;
  crt_basis b;
  if (crt_basis_init(&b, primes, limbs)) {
    crt_basis_free(&b);
    return -1;
  }
  uint64_t ql = primes[limbs - 1];
  big_t half;
  big_set_u64(&half, mode ? ql / 2 : 0);
  for (uint64_t bi = 0; bi < batch; ++bi)
    for (uint64_t e = 0; e < n; ++e) {
      big_t X, Y;
      crt_value(&b, in + bi * limbs * n + e, n, &X); /* X in [0, prod q) */
      big_add(&X, &half);
      big_div_u64(&Y, &X, ql); /* floor */
      for (uint32_t l = 0; l + 1 < limbs; ++l) out[(bi * (limbs - 1) + l) * n + e] = big_mod_u64(&Y, primes[l]);
    }
  crt_basis_free(&b);
  return 0;
}

/* ---- modraise ---------------------------------------------------------------- */

int orc_modraise(uint64_t *out, const uint64_t *in, uint64_t batch, uint32_t from, uint32_t to, uint64_t n,
                 const uint64_t *primes) {
  if (from == 0 || to <= from) return -1;
  for (uint64_t bi = 0; bi < batch; ++bi)
    orc_basis_extend(in + bi * from * n, from, primes, out + bi * to * n, to, primes, n);
  return 0;
}
