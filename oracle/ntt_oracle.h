/*
 * ntt_oracle.h -- plain C reference ("oracle") for batched RNS negacyclic NTT,
 * pointwise products, Galois automorphisms and the hybrid rotation key-switch.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is slow and obviously correct by
 * construction; it exists so that the GPU library can be checked against it bit
 * for bit.  Only the test-suite, the smoke check and the CPU-baseline leg of the
 * benchmark load it.  It shares no source, header, table or constant generator
 * with the GPU library.
 *
 * Arithmetic: every modular product is `(unsigned __int128)a * b % q`; there is
 * no Shoup, Montgomery or Barrett step anywhere in this file's implementation.
 * Multi-prime reconstructions use explicit multi-word integers.
 *
 * What the pages fix and what is a reading:
 *   - The kestrel-llm data-flow overview (lpnh.cn, section 3, "four layers of
 *     the ciphertext side") names the negacyclic NTT + polynomial multiply as the
 *     bottom arithmetic layer and proves it bit-exact against the textbook O(n^2)
 *     transform; this oracle follows that practice.
 *   - FHElium "Eager, Compile, and native execution", section "CUDA execution",
 *     lists the kernel families reproduced here: coefficient-wise RNS products,
 *     mixed-radix decomposition and basis extension, NTT, Galois automorphisms,
 *     key-switch multiply-accumulate and QP-to-Q ModDown; section "Shared
 *     implementation and native path" fixes the [*batch, limb, coefficient]
 *     layout with limb j using modulus j.
 *   - Everything the pages leave open (choice of psi, output order, digit
 *     partition, exact vs approximate basis extension, floor ModDown, output
 *     ranges) follows the readings stated next to each function below.
 */
#ifndef NTT_ORACLE_H
#define NTT_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- number theory ------------------------------------------------------ */

/* Deterministic Miller-Rabin with the first twelve prime bases (2..37): exact
 * for every n < 3.3e24, hence for all 64-bit n. Returns 1 if prime. */
int orc_is_prime(uint64_t n);

/* The first `count` primes q below 2^bits, in descending order, with
 * q == 1 (mod two_n).  Returns the number found (== count on success). */
uint32_t orc_find_primes(uint32_t bits, uint64_t two_n, uint32_t count, uint64_t *out);

/* psi: the smallest x in [2, q) with x^n == -1 (mod q) (a primitive 2n-th root
 * of unity; n a power of two).  Returns 0 if q has no such root. */
uint64_t orc_find_psi(uint64_t q, uint64_t n);

uint64_t orc_pow_mod(uint64_t b, uint64_t e, uint64_t q);
uint64_t orc_inv_mod(uint64_t a, uint64_t q); /* q prime, a != 0 mod q */

/* ---- single-limb transforms over Z_q[X]/(X^n + 1) ------------------------ */

/* Definition (O(n^2)): out[k] = sum_i a[i] * psi^((2*brv(k)+1)*i) mod q, i.e. the
 * evaluation of a at psi^(2*brv(k)+1), stored in bit-reversed order of the odd
 * exponents.  n = 2^m. */
void orc_ntt_definition(const uint64_t *a, uint64_t *out, uint64_t n, uint64_t q, uint64_t psi);
/* Definition of the inverse: a[i] = n^-1 * sum_k ahat[k] * psi^-((2*brv(k)+1)*i). */
void orc_intt_definition(const uint64_t *ahat, uint64_t *out, uint64_t n, uint64_t q, uint64_t psi);

/* Textbook in-place radix-2 transforms computing exactly the two definitions
 * above (decimation in time with the psi^brv table, decimation in frequency
 * with the psi^-brv table, then scaling by n^-1).  Input and output canonical. */
void orc_ntt_forward(uint64_t *a, uint64_t n, uint64_t q, uint64_t psi);
void orc_ntt_inverse(uint64_t *a, uint64_t n, uint64_t q, uint64_t psi);

/* Schoolbook negacyclic product c = a*b mod (X^n + 1, q), O(n^2). */
void orc_negacyclic_schoolbook(const uint64_t *a, const uint64_t *b, uint64_t *c, uint64_t n, uint64_t q);

/* Coefficient-domain automorphism sigma_g: X -> X^g (g odd):
 * for each i, e = i*g mod 2n; out[e] = in[i] if e < n else out[e-n] = -in[i]. */
void orc_automorph_coeff(const uint64_t *in, uint64_t *out, uint64_t n, uint64_t q, uint64_t g);
/* NTT-domain automorphism: out[k] = in[p(k)] with 2*brv(p(k))+1 == (2*brv(k)+1)*g mod 2n,
 * so that NTT(sigma_g(a)) == orc_automorph_ntt(NTT(a)). */
void orc_automorph_ntt(const uint64_t *in, uint64_t *out, uint64_t n, uint64_t g);

/* ---- batched [batch][limbs][n] drivers ----------------------------------- */
/* Tensor limb t (0 <= t < limbs) uses primes[t]; psi per prime by orc_find_psi.
 * `threads` <= 0 means one. Returns 0, or -1 if a prime has no psi. */
int orc_batch_ntt(uint64_t *data, uint64_t batch, uint32_t limbs, uint64_t n, const uint64_t *primes,
                  int inverse, int threads);
/* out = a*b element-wise, mod the limb's prime. out may alias a or b. */
void orc_batch_pointwise(uint64_t *out, const uint64_t *a, const uint64_t *b, uint64_t batch, uint32_t limbs,
                         uint64_t n, const uint64_t *primes);
/* Ciphertext tensor product on [batch][2][limbs][n] pairs -> [batch][3][limbs][n]:
 * d0 = a0 b0, d1 = a0 b1 + a1 b0, d2 = a1 b1 (mod q). */
void orc_batch_tensor(uint64_t *out, const uint64_t *a, const uint64_t *b, uint64_t batch, uint32_t limbs,
                      uint64_t n, const uint64_t *primes);
/* domain 0 = coefficient, 1 = NTT (bit-reversed). */
void orc_batch_automorph(uint64_t *out, const uint64_t *in, uint64_t g, int domain, uint64_t batch,
                         uint32_t limbs, uint64_t n, const uint64_t *primes);

/* ---- key-switch pieces ---------------------------------------------------- */
/* Basis extension of one digit.  x: [k][n] residues modulo src[0..k); the value of
 * coefficient e is the unique D in [0, prod src) with D == x[t][e] mod src[t]
 * (exact CRT, unsigned representative).  out: [m][n] with out[t][e] = D mod dst[t]. */
void orc_basis_extend(const uint64_t *x, uint32_t k, const uint64_t *src, uint64_t *out, uint32_t m,
                      const uint64_t *dst, uint64_t n);

/* Exact floor ModDown from Q*P to Q. acc: [nq+np][n] (limbs of Q then of P, all
 * coefficient domain); out: [nq][n] with out[l][e] = floor(X_e / P) mod q_l where
 * X_e in [0, QP) is the CRT value of column e. */
void orc_moddown(const uint64_t *acc, uint64_t *out, const uint64_t *qp, uint32_t nq, uint32_t np, uint64_t n);

/* Hybrid rotation key-switch of a batch of ciphertexts.
 *  ct, out: [batch][2][nq][n], coefficient domain, canonical residues mod q_l.
 *  ksk:     [dnum][2][nq+np][n], NTT domain over the basis qp = Q ++ P.
 *  Steps (in the order the large-ring key-switch workload lists them):
 *    c' = sigma_g(c) for both components;
 *    digit j = limbs [j*a, (j+1)*a) of c1', a = nq/dnum;
 *    D_j = exact CRT of digit j, reduced onto all nq+np primes (basis extension);
 *    NTT of every extended digit;
 *    acc_c = sum_j NTT(D_j) * ksk[j][c] (per limb, mod its prime);
 *    INTT of acc_c;
 *    ModDown (exact floor) of acc_c to Q;
 *    out = (c0' + ModDown(acc_0), ModDown(acc_1)).
 * Returns 0, or -1 on a bad argument. */
int orc_keyswitch(uint64_t *out, const uint64_t *ct, const uint64_t *ksk, uint64_t g, uint64_t batch,
                  uint64_t n, const uint64_t *qp, uint32_t nq, uint32_t np, uint32_t dnum, int threads);

/* Hoisted rotations: R Galois elements share one decomposition of c1 (the
 * rotate_k / conj_extract / coeff_to_slot stages of the kestrel-llm overview,
 * section 4.2, apply many rotations, and the conjugation g = 2n - 1, to one
 * ciphertext).
 *  ct:  [batch][2][nq][n] coefficient domain;  gs: R odd Galois elements < 2n;
 *  ksk: [R][dnum][2][nq+np][n] NTT domain (key r carries sigma_{g_r}(s) to s);
 *  out: [R][batch][2][nq][n].
 *  Steps: digits of c1 WITHOUT the automorphism, exact CRT lift, reduced onto Q u P;
 *  NTT of every extended digit (once); then for each r: the NTT-domain automorphism
 *  of every extended limb (the slot permutation of orc_automorph_ntt), the inner
 *  product with ksk[r], INTT, ModDown (exact floor), and sigma_{g_r}(c0) added to
 *  component 0.  The digits are then sigma_g of the lifted integers, which differ
 *  from the lifts of sigma_g(c1) where a coefficient changes sign; both are valid
 *  decompositions (same congruence, same size bound), so this is its own result,
 *  not orc_keyswitch's.  Returns 0, or -1 on a bad argument. */
int orc_keyswitch_hoisted(uint64_t *out, const uint64_t *ct, const uint64_t *ksk, const uint64_t *gs, uint32_t R,
                          uint64_t batch, uint64_t n, const uint64_t *qp, uint32_t nq, uint32_t np, uint32_t dnum,
                          int threads);

/* Relinearisation of a batch of tensor products d = (d0, d1, d2), each
 * [batch][3][nq][n] in the coefficient domain: the quadratic term is switched with
 * the relinearisation key rlk [dnum][2][nq+np][n] (NTT domain over Q u P), with no
 * automorphism (g = 1):  out = (d0 + ModDown(acc_0), d1 + ModDown(acc_1)),
 * acc_c = INTT(sum_j NTT(ModUp(digit_j(d2))) * rlk[j][c]).  out: [batch][2][nq][n].
 * The kestrel-llm overview (section 3) lists relin beside mul and rescale in its
 * CKKS layer.  Returns 0, or -1 on a bad argument. */
int orc_relinearize(uint64_t *out, const uint64_t *d, const uint64_t *rlk, uint64_t batch, uint64_t n,
                    const uint64_t *qp, uint32_t nq, uint32_t np, uint32_t dnum, int threads);

/* Rescale by the last prime of a basis (FHElium "Eager, Compile, and native
 * execution", section "CUDA execution": nearest and truncating rescale kernels).
 * in: [batch][limbs][n] coefficient domain modulo primes[0..limbs); X = the CRT
 * value of a column in [0, prod primes).  out: [batch][limbs-1][n] with
 *   mode 0 (truncating): out[l] = floor(X / q_last) mod q_l,
 *   mode 1 (nearest):    out[l] = floor((X + floor(q_last / 2)) / q_last) mod q_l.
 * Returns 0, or -1 on a bad argument. */
int orc_rescale(uint64_t *out, const uint64_t *in, int mode, uint64_t batch, uint32_t limbs, uint64_t n,
                const uint64_t *primes);

/* ModRaise: kestrel-llm data-flow overview, section 4.2 (the modraise stage that
 * opens the bootstrapping profile).  Each coefficient is lifted to its exact
 * integer on the first `from` primes and re-reduced onto the longer chain.
 * in: [batch][from][n] coefficient domain modulo primes[0..from); out:
 * [batch][to][n] modulo primes[0..to), to > from: out[t] = X mod primes[t] with X the
 * exact CRT value of the column in [0, prod_{i<from} primes[i]) (the unsigned
 * representative that Garner's mixed-radix reconstruction yields).  The first
 * `from` output limbs equal the input.  Returns 0, or -1 on a bad argument. */
int orc_modraise(uint64_t *out, const uint64_t *in, uint64_t batch, uint32_t from, uint32_t to, uint64_t n,
                 const uint64_t *primes);

/* Multi-word CRT helper exposed for tests: value of residues x[0..k) modulo
 * m[0..k) as little-endian 64-bit words into out (capacity `words`).  Returns the
 * number of significant words, or -1 if it does not fit. */
int orc_crt_words(const uint64_t *x, const uint64_t *m, uint32_t k, uint64_t *out, uint32_t words);

#ifdef __cplusplus
}
#endif
#endif
