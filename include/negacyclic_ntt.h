/*
 * negacyclic_ntt.h -- C ABI of the MI355X (gfx950) negacyclic NTT library.
 *
 * What it computes (all integer arithmetic, results bit-exact and independent
 * of launch configuration):
 *   - batched RNS negacyclic NTT / inverse NTT over Z_q[X]/(X^n + 1);
 *   - pointwise modular products and the ciphertext tensor product in the NTT
 *     domain;
 *   - Galois automorphisms X -> X^g (coefficient domain and NTT domain, and fused
 *     into the forward transform);
 *   - the hybrid rotation key-switch: automorphism, digit decomposition, exact
 *     basis extension (ModUp), NTT, key inner product, inverse NTT, ModDown.
 * These are the RNS/NTT kernel families FHElium lists for its native layer
 * ("Eager, Compile, and native execution", section "CUDA execution": Montgomery
 * products, mixed-radix decomposition and basis extension, NTT, Galois
 * automorphisms, key-switch multiply-accumulate, QP-to-Q ModDown), and the
 * negacyclic NTT + polynomial product layer of the kestrel-llm engine (lpnh.cn
 * data-flow overview, section 3), whose rotation key-switches dominate the
 * coeff_to_slot / slot_to_coeff stages (section 4.2).
 *
 * Conventions (all entry points):
 *   Layout.   An RNS tensor is a dense row-major array [batch][limb][n] of
 *             uint64 residues, coefficient (or NTT slot) fastest; tensor limb t
 *             uses modulus limb_begin + t of the plan (FHElium, section "Shared
 *             implementation and native path": shape [*batch, limb, coefficient],
 *             parameter column j describes limb j).
 *   Domains.  Coefficient domain: a[i] is the coefficient of X^i.  NTT domain:
 *             slot k holds a(psi^(2*brv(k)+1)) mod q, brv = bit reversal of
 *             log2(n) bits, psi = the plan's primitive 2n-th root of unity.
 *   Ranges.   Inputs must be canonical (< q); outputs are always canonical
 *             (FHElium, section "One operation through both use models": standard
 *             RNS results lie in [0, q_i)).  Non-canonical input gives an
 *             unspecified (but in-bounds) result.
 *   Memory.   Every data pointer is a device pointer owned by the caller (the
 *             library never allocates or frees on the call path); plans own their
 *             device tables.  Mixed devices are the caller's error.
 *   Streams.  `stream` is a hipStream_t (NULL = the device's null stream).  Work
 *             is enqueued on it and the call returns without synchronising, so
 *             device faults surface at the caller's next synchronisation
 *             (FHElium, section "CUDA execution").  A stable address does not mean
 *             a completed use: callers order buffer reuse with events (FHElium,
 *             "Value signatures and reusable buffers", section "The writer cannot
 *             infer arbitrary readers").
 *   Errors.   Arguments are validated before anything is launched (FHElium,
 *             section "Schema registration and device dispatch"): NTT_EINVAL,
 *             NTT_EUNSUPPORTED and NTT_EOVERLAP mean nothing was enqueued.
 *             NTT_EDEVICE also reports a failed launch; launches of the same call
 *             that preceded it (a call may take several) stay enqueued.
 *   Threads.  Plans are immutable after creation; concurrent calls on different
 *             streams are safe when their output and workspace buffers differ.
 */
#ifndef NEGACYCLIC_NTT_H
#define NEGACYCLIC_NTT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NTT_OK = 0,
  NTT_EINVAL = -1,       /* bad argument: size, prime, range, null pointer, misalignment */
  NTT_EUNSUPPORTED = -2, /* valid but outside what this build implements */
  NTT_ENOMEM = -3,       /* plan tables could not be allocated */
  NTT_EDEVICE = -4,      /* HIP runtime error (device selection, copy or launch) */
  NTT_EOVERLAP = -5      /* forbidden aliasing between output and inputs */
} ntt_status;

typedef struct ntt_plan ntt_plan;       /* opaque: n, primes, tables; immutable */
typedef struct ntt_ks_plan ntt_ks_plan; /* opaque: key-switch constants; immutable */
typedef struct ntt_mr_plan ntt_mr_plan; /* opaque: modraise constants; immutable */

/* Human-readable name of a status code (static string).  Errors are reported
 * before launch, as FHElium validates before dispatch ("Eager, Compile, and
 * native execution", section "Schema registration and device dispatch"). */
const char *ntt_status_string(int status);

/* Host utility: the first `count` primes q below 2^bits with q == 1 (mod 2n), in
 * descending order, written to out[0..count).  bits in [3, 62], n a power of two
 * in [2, 2^16].  NTT_EINVAL if fewer than `count` exist.  The moduli are a
 * caller-side parameter (FHElium "Eager, Compile, and native execution", section
 * "Execution properties": modulus parameters enter native execution as arguments);
 * this helper only picks the NTT-friendly ones the workloads use. */
int ntt_find_primes(uint32_t bits, uint32_t n, uint32_t count, uint64_t *out);

/* Create a plan for ring degree n (a power of two, 2 <= n <= 65536) and the
 * moduli primes[0..num_primes) (host array, copied).  The plan holds what FHElium
 * passes to its native NTT as tensors -- modulus parameters and twiddle tables
 * ("Eager, Compile, and native execution", section "Execution properties";
 * section "Shared implementation and native path": parameter column j describes
 * limb j) -- built once and kept on the device.  Each prime must satisfy
 * 3 <= q < 2^62, q == 1 (mod 2n), be prime (deterministic Miller-Rabin) and be
 * distinct from the others.  psi: optional host array of one primitive 2n-th
 * root per prime (psi^n == -1 mod q); NULL selects, per prime, the smallest
 * x >= 2 with x^n == -1.  The plan precomputes, per prime, the bit-reversed
 * tables psi^brv(k) and psi^-brv(k) with their Shoup companions
 * floor(w * 2^64 / q) (and floor(w * 2^32 / q) for primes below 2^30), and n^-1.
 * device >= 0 uploads them to that HIP device; device == -1 builds a host-only
 * plan usable with ntt_plan_get_tables but rejected (NTT_EDEVICE) by every
 * compute call.  *out receives the plan (NULL on error). */
int ntt_plan_create(ntt_plan **out, uint32_t n, const uint64_t *primes, uint32_t num_primes, const uint64_t *psi,
                    int device);

/* Host copies of one prime's tables (each array n entries; any pointer may be
 * NULL to skip it): fwd[k] = psi^brv(k), fwd_shoup[k] = floor(fwd[k]*2^64/q),
 * inv[k] = psi^-brv(k), inv_shoup likewise.  *psi_out (nullable) gets psi.  These
 * are the NTT and inverse tables of FHElium's native calls ("Eager, Compile, and
 * native execution", section "Shared implementation and native path"), exposed
 * so that callers and tests can check them.  NTT_EINVAL for limb >= num_primes. */
int ntt_plan_get_tables(const ntt_plan *plan, uint32_t limb, uint64_t *psi_out, uint64_t *fwd, uint64_t *fwd_shoup,
                        uint64_t *inv, uint64_t *inv_shoup);

/* n, number of primes and prime `limb` of a plan (for bindings): the parameter
 * columns of FHElium's limb layout ("Eager, Compile, and native execution",
 * section "Shared implementation and native path").  NTT_EINVAL on a NULL plan or
 * an out-of-range limb. */
int ntt_plan_info(const ntt_plan *plan, uint32_t *n, uint32_t *num_primes, int *device);
int ntt_plan_prime(const ntt_plan *plan, uint32_t limb, uint64_t *q);

/* Release a plan.  The caller guarantees no enqueued work still uses it: a
 * stable address is not a completed use (FHElium, "Value signatures and reusable
 * buffers", section "The writer cannot infer arbitrary readers"). */
void ntt_plan_destroy(ntt_plan *plan);

/* Forward negacyclic NTT, in place, on data[batch][num_limbs][n] (coefficient
 * domain in, bit-reversed NTT domain out).  Limb t uses prime limb_begin + t.
 * data must be 16-byte aligned.  The kestrel-llm overview (section 3) names this
 * transform as the bottom arithmetic layer; the pages give no formula, so the
 * definition in the "Domains" convention above is the contract. */
int ntt_forward(const ntt_plan *plan, uint64_t *data, uint64_t batch, uint32_t limb_begin, uint32_t num_limbs,
                void *stream);

/* Inverse of ntt_forward, in place, including the n^-1 scaling (so that
 * ntt_inverse(ntt_forward(a)) == a): the inverse transform whose tables FHElium
 * passes to its native NTT ("Eager, Compile, and native execution", section
 * "Shared implementation and native path": NTT tables and inverse tables).  Same
 * layout, alignment and errors as ntt_forward. */
int ntt_inverse(const ntt_plan *plan, uint64_t *data, uint64_t batch, uint32_t limb_begin, uint32_t num_limbs,
                void *stream);

/* Forward NTT of sigma_g(in): out = NTT(in(X^g)) with the automorphism folded
 * into the transform (no separate pass over memory).  galois_elt odd and
 * < 2n (1 gives the plain forward NTT).  out may equal in exactly (in place);
 * partial overlap -> NTT_EOVERLAP.  FHElium lists Galois automorphisms among
 * its native CKKS primitives ("Eager, Compile, and native execution", section
 * "CUDA execution"). */
int ntt_forward_galois(const ntt_plan *plan, uint64_t *out, const uint64_t *in, uint64_t galois_elt, uint64_t batch,
                       uint32_t limb_begin, uint32_t num_limbs, void *stream);

/* Pointwise product out = a * b mod q_limb (NTT domain; FHElium, section "CUDA
 * execution": coefficient-wise RNS multiplication).  out may equal a or b
 * exactly; partial overlap -> NTT_EOVERLAP. */
int poly_mul_ntt(const ntt_plan *plan, uint64_t *out, const uint64_t *a, const uint64_t *b, uint64_t batch,
                 uint32_t limb_begin, uint32_t num_limbs, void *stream);

/* Ciphertext tensor product in the NTT domain: a, b are [batch][2][num_limbs][n],
 * out is [batch][3][num_limbs][n] with d0 = a0 b0, d1 = a0 b1 + a1 b0,
 * d2 = a1 b1 (mod q).  The ciphertext "mul" of the kestrel-llm CKKS layer
 * (section 3).  out must not overlap a or b (NTT_EOVERLAP). */
int ct_tensor_ntt(const ntt_plan *plan, uint64_t *out, const uint64_t *a, const uint64_t *b, uint64_t batch,
                  uint32_t limb_begin, uint32_t num_limbs, void *stream);

/* Ciphertext product in the coefficient domain, for n <= 4096: a, b are
 * [batch][2][num_limbs][n] coefficient-domain ciphertexts; out is
 * [batch][3][num_limbs][n] with the negacyclic products (in Z_q[X]/(X^n + 1))
 *   d0 = a0 b0,  d1 = a0 b1 + a1 b0,  d2 = a1 b1,
 * i.e. INTT(ct_tensor_ntt(NTT(a), NTT(b))), computed in one launch that keeps each
 * (ciphertext, limb) in LDS through the four forward transforms, the slot products
 * and the three inverse transforms.  This is the ciphertext "mul" of the kestrel-llm
 * CKKS layer (section 3) on its inner-chain shape (section 5: n = 2048, 112 primes,
 * 4 token positions x 2 components).  out must not overlap a or b (NTT_EOVERLAP);
 * n > 4096 is NTT_EUNSUPPORTED (use ntt_forward, ct_tensor_ntt, ntt_inverse). */
int ct_tensor_coeff(const ntt_plan *plan, uint64_t *out, const uint64_t *a, const uint64_t *b, uint64_t batch,
                    uint32_t limb_begin, uint32_t num_limbs, void *stream);

/* Galois automorphism sigma_g: X -> X^g, galois_elt odd and < 2n.
 * domain 0 (coefficient): out[i*g mod 2n] = in[i] when i*g mod 2n < n, else
 *   out[i*g mod 2n - n] = -in[i] (a signed permutation).
 * domain 1 (NTT): out[k] = in[p(k)] with 2 brv(p(k)) + 1 == (2 brv(k) + 1) g
 *   (mod 2n), so that automorph(NTT(a), 1) == NTT(automorph(a, 0)).
 * out must not overlap in (NTT_EOVERLAP).  The rotate_k / coeff_to_slot stages
 * of kestrel-llm (section 4.2) apply these rotations. */
int automorph(const ntt_plan *plan, uint64_t *out, const uint64_t *in, uint64_t galois_elt, int domain,
              uint64_t batch, uint32_t limb_begin, uint32_t num_limbs, void *stream);

/* Rescale by the last prime of a limb range (FHElium "Eager, Compile, and native
 * execution", section "CUDA execution": nearest and truncating rescale kernels;
 * "rescale" of the kestrel-llm overview's CKKS layer, section 3).
 *   in  : [batch][num_limbs][n], coefficient domain, canonical residues modulo the
 *         plan primes [limb_begin, limb_begin + num_limbs); num_limbs >= 2;
 *   out : [batch][num_limbs - 1][n] modulo the same primes without the last one,
 *         q_k = prime (limb_begin + num_limbs - 1).  With X in [0, prod q) the CRT
 *         value of a coefficient's residues:
 *           mode 0 (truncating): out = floor(X / q_k)              mod q_l,
 *           mode 1 (nearest):    out = floor((X + floor(q_k / 2)) / q_k) mod q_l.
 * Exact integer arithmetic, so bit-exact.  out must not overlap in (NTT_EOVERLAP);
 * mode other than 0 / 1 or num_limbs < 2 is NTT_EINVAL. */
int rescale(const ntt_plan *plan, uint64_t *out, const uint64_t *in, int mode, uint64_t batch, uint32_t limb_begin,
            uint32_t num_limbs, void *stream);

/* ---- input checks (debugging) -------------------------------------------- */

/* Adds to *count (a device uint64, 8-byte aligned, zeroed by the caller) the number of
 * residues of data [batch][num_limbs][n] that are not canonical, i.e. >= the plan
 * prime of their limb (limb_begin + t).  Asynchronous on `stream`.  Every other entry
 * point assumes canonical inputs (outputs of non-canonical inputs are unspecified
 * but every access stays in bounds). */
int ntt_count_noncanonical(const ntt_plan *plan, const uint64_t *data, uint64_t batch, uint32_t limb_begin,
                           uint32_t num_limbs, uint64_t *count, void *stream);

/* Debug mode (off unless the environment variable NTT_CHECK_INPUTS is set to a value
 * other than "" or "0"; this call overrides it for the process): every entry point
 * first counts the non-canonical residues of its inputs -- operands, ciphertexts and
 * keys -- waits for the count on the caller's stream and returns NTT_EINVAL, having
 * launched nothing else, if any is found.  The checks synchronise the stream and are
 * serialised across threads; the FHElium pages ("Eager, Compile, and native
 * execution", section "Schema registration and device dispatch") validate inputs
 * before any launch, and this extends that to the values, at a cost. */
void ntt_set_debug_checks(int on);

/* Threads per kernel launch.  A dispatch packet holds at most 2^32 - 1 work-items
 * per grid dimension, so calls whose grid would exceed the cap are split into
 * several launches of whole polynomials (whole ciphertexts for ct_tensor_ntt), in
 * order, on the caller's stream.  threads = 0 restores the default cap,
 * 2^32 - 2^16; a smaller cap (at least 256) makes the splitting testable at small
 * sizes.  Process-wide; NTT_EINVAL for 1..255.  A single polynomial whose
 * launch alone exceeds the cap is NTT_EUNSUPPORTED. */
int ntt_set_max_launch_threads(uint64_t threads);

/* Key-switch plan over a Q u P basis (the basis-extension and ModDown constants
 * of FHElium's key-switch, "Eager, Compile, and native execution", section "CUDA
 * execution"; they enter native execution as arguments, section "Execution
 * properties"): the first num_q primes of qp_plan form Q
 * and the next num_p form P (num_q + num_p <= primes in qp_plan); Q is split into
 * dnum digits of num_q / dnum consecutive primes (num_q % dnum == 0,
 * num_q / dnum <= 16, num_p <= 16).  Precomputes the Garner (mixed-radix)
 * constants of every digit and of P, the products of each digit's and of P's
 * primes modulo every target prime, and P^-1 mod q.  qp_plan must be a device
 * plan and must outlive this plan. */
int keyswitch_plan_create(ntt_ks_plan **out, const ntt_plan *qp_plan, uint32_t num_q, uint32_t num_p,
                          uint32_t dnum);

/* Bytes of device workspace keyswitch (and relinearize) need for `batch`
 * ciphertexts.  The caller allocates it: FHElium leaves allocation to the caller's
 * allocator ("Eager, Compile, and native execution", section "Execution
 * properties").  NTT_EUNSUPPORTED for batch > 4096. */
int keyswitch_workspace_size(const ntt_ks_plan *plan, uint64_t batch, size_t *bytes);

/* Rotation key-switch (hybrid, dnum digits):
 *   ct, out : [batch][2][num_q][n], coefficient domain;
 *   ksk     : [dnum][2][num_q + num_p][n], NTT domain over Q u P (limbs Q then P;
 *             component 0 pairs with the c0 accumulator);
 *   out = ( sigma_g(c0) + ModDown(acc_0), ModDown(acc_1) ) where
 *   acc_c = INTT( sum_j NTT(ModUp(digit_j(sigma_g(c1)))) * ksk[j][c] ).
 * ModUp is exact: digit j's residues are lifted to the unique integer in
 * [0, Q_j) (mixed-radix / Garner, the "mixed-radix decomposition and basis
 * extension" and "Garner extension" named by FHElium, section "CUDA execution",
 * and kestrel-llm, section 4.2) and reduced onto every other prime.  ModDown is
 * the exact floor: out = floor(X / P) mod q for the integer X in [0, QP) with
 * the accumulator's residues (FHElium's "QP-to-Q ModDown").
 * galois_elt odd and < 2n (1 = no rotation, a plain key-switch).  batch <= 4096
 * (NTT_EUNSUPPORTED beyond).  workspace: device buffer of at least
 * keyswitch_workspace_size bytes, 256-byte aligned, not overlapping out/ct/ksk.
 * out must not overlap ct, ksk or workspace. */
int keyswitch(const ntt_ks_plan *plan, uint64_t *out, const uint64_t *ct, const uint64_t *ksk,
              uint64_t galois_elt, uint64_t batch, void *workspace, size_t workspace_bytes, void *stream);

/* keyswitch() for callers that cannot allocate device memory on the call path
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation, arguments, layouts and errors as keyswitch(),
 * with the workspace taken from a static device array of the library instead of a
 * caller buffer.  The array holds 80 MiB (83,886,080 bytes) per GPU -- one
 * ciphertext at n = 2^16 over 24 + 8 primes with 3 digits -- and a call whose
 * keyswitch_workspace_size exceeds it returns NTT_EUNSUPPORTED with nothing
 * launched.  A GPU holds the array from the first call on it until the process
 * ends.  Every call on one GPU uses that GPU's one array: calls that overlap on a
 * GPU (concurrent streams, or threads) race on it and must be ordered by the
 * caller.  Nothing needs to start at zero: each call writes every workspace byte
 * it reads.  Allocates nothing and never synchronises (debug checks aside). */
int keyswitch_noalloc(const ntt_ks_plan *plan, uint64_t *out, const uint64_t *ct, const uint64_t *ksk,
                      uint64_t galois_elt, uint64_t batch, void *stream);

/* Bytes of device workspace keyswitch_hoisted needs for num_rot rotations of `batch`
 * ciphertexts: batch * ((dnum + 2 num_rot) * (num_q + num_p) + num_q) * n * 8 (caller-owned,
 * as for keyswitch_workspace_size).  NTT_EINVAL for num_rot 0, NTT_EUNSUPPORTED for
 * num_rot > 64 or batch > 4096. */
int keyswitch_hoisted_workspace_size(const ntt_ks_plan *plan, uint32_t num_rot, uint64_t batch, size_t *bytes);

/* Hoisted rotations: num_rot Galois elements applied to the same ciphertexts with
 * ONE decomposition (ModUp and forward NTT of c1 once, then per rotation the
 * NTT-domain automorphism of the shared digits -- a slot permutation fused into the
 * key product -- INTT and ModDown).  The rotate_k, conj_extract (g = 2n - 1) and
 * coeff_to_slot stages of the kestrel-llm overview, section 4.2, apply many
 * rotations to one ciphertext.
 *   ct          : [batch][2][num_q][n], coefficient domain;
 *   ksk         : [num_rot][dnum][2][num_q + num_p][n], key r for galois_elts[r];
 *   galois_elts : HOST array of num_rot odd elements < 2n (1 <= num_rot <= 64);
 *   out         : [num_rot][batch][2][num_q][n];
 *   out[r] = ( sigma_g(c0) + ModDown(acc_0), ModDown(acc_1) ),
 *   acc_c = INTT( sum_j slot_g(NTT(ModUp(digit_j(c1)))) * ksk[r][j][c] ).
 * The digits are sigma_g of the lifted digits of c1, not the lifts of
 * sigma_g(c1): where sigma_g flips a coefficient's sign they differ by the digit
 * modulus, so the result differs from keyswitch() by a valid re-encryption of the
 * same value (both decompositions satisfy the same congruence and bound).
 * dnum <= 16, batch <= 4096.  workspace: keyswitch_hoisted_workspace_size bytes,
 * 256-byte aligned.  out must not overlap ct, ksk or workspace. */
int keyswitch_hoisted(const ntt_ks_plan *plan, uint64_t *out, const uint64_t *ct, const uint64_t *ksk,
                      const uint64_t *galois_elts, uint32_t num_rot, uint64_t batch, void *workspace,
                      size_t workspace_bytes, void *stream);

/* Relinearisation of tensor products (the "relin" operation of the kestrel-llm
 * overview's CKKS layer, section 3; it closes the ciphertext-ciphertext multiply
 * whose tensor step is ct_tensor_ntt):
 *   d   : [batch][3][num_q][n], coefficient domain (d0, d1, d2);
 *   rlk : [dnum][2][num_q + num_p][n], NTT domain over Q u P, the key that carries
 *         s^2 to s (same layout as a rotation key);
 *   out : [batch][2][num_q][n] = ( d0 + ModDown(acc_0), d1 + ModDown(acc_1) ) with
 *         acc_c = INTT( sum_j NTT(ModUp(digit_j(d2))) * rlk[j][c] ).
 * The same ModUp / key product / ModDown as keyswitch with no automorphism.
 * batch <= 4096.  workspace: as for keyswitch (keyswitch_workspace_size bytes for
 * `batch`).  out must not overlap d, rlk or workspace (NTT_EOVERLAP). */
int relinearize(const ntt_ks_plan *plan, uint64_t *out, const uint64_t *d, const uint64_t *rlk, uint64_t batch,
                void *workspace, size_t workspace_bytes, void *stream);

/* Release a key-switch plan (caller guarantees no enqueued use, as for
 * ntt_plan_destroy). */
void keyswitch_plan_destroy(ntt_ks_plan *plan);

/* ---- ModRaise ------------------------------------------------------------ */

/* ModRaise plan: lift from the first num_from primes of `plan` to its first num_to
 * (num_from < num_to <= primes in plan, num_from <= 16).  Precomputes the Garner
 * constants of the source primes and their products modulo every target.  `plan`
 * must be a device plan and must outlive this plan. */
int modraise_plan_create(ntt_mr_plan **out, const ntt_plan *plan, uint32_t num_from, uint32_t num_to);

/* ModRaise: kestrel-llm data-flow overview, section 4.2 (the modraise stage that
 * opens the bootstrapping profile).  Each coefficient's residues on the first
 * num_from primes are lifted to their exact integer and re-reduced onto the longer
 * chain.
 *   in  : [batch][num_from][n], coefficient domain;
 *   out : [batch][num_to][n]: out[t] = X mod q_t with X in [0, q_0 ... q_{from-1})
 *         the exact CRT value of the column (Garner's unsigned representative); the
 *         first num_from limbs equal the input.
 * out must not overlap in (NTT_EOVERLAP). */
int modraise(const ntt_mr_plan *plan, uint64_t *out, const uint64_t *in, uint64_t batch, void *stream);

/* Release a ModRaise plan (caller guarantees no enqueued use, as for
 * ntt_plan_destroy). */
void modraise_plan_destroy(ntt_mr_plan *plan);

#ifdef __cplusplus
}
#endif
#endif
