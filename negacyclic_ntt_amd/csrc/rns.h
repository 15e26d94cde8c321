// Residue-number-system device helpers for gfx950: Shoup products by plan constants,
// Garner's mixed-radix digits, their evaluation modulo other primes (plain Shoup
// sums, or the 30-bit-half dot product below 2^60), the coefficient-domain
// automorphism gather and the device constants of a key-switch plan.  Shared by
// the key-switch kernels (keyswitch.hip) and the transform passes they fuse into.
#pragma once
#include "internal.h"

namespace nntt {
namespace {

constexpr int kMaxDigitPrimes = 16;  // table row strides of the device constants
constexpr int kMaxSpecial = 16;

using Tw = Wide::Tw;

// Shoup product by a plan constant {w, floor(w 2^64 / q)}.  When every prime of the
// plan is below 2^60 (B60), the 2^62-scaled companion floor(floor(w 2^64/q) / 4) is
// used with the cheaper carry-free quotient (see Wide60); the shift is on a uniform
// constant, so it runs on the scalar unit.
template <bool B60>
__device__ __forceinline__ uint64_t shoup(uint64_t y, Tw c, uint64_t q) {
  if constexpr (B60) return Wide60::mul(y, Wide60::Tw{c.w, c.wp >> 2}, q);
  else return Wide::mul(y, c, q);
}

// acc, t in [0, 2q) -> (acc + t) in [0, 2q).  Below 2^60 the sum stays below 2^62,
// so the compare-free sign select applies.
template <bool B60>
__device__ __forceinline__ uint64_t lazy_add(uint64_t acc, uint64_t t, uint64_t two_q) {
  if constexpr (B60) return csub_sign(acc + t, two_q);
  else return csub(acc + t, two_q);
}

// Garner digits of k residues (k <= K, runtime).  m[i] the moduli, g[i * S + k]
// (S = table row stride) holds prod_{j<k} m_j mod m_i for k < i and
// (prod_{j<i} m_j)^-1 mod m_i at k = i.  Output v[i] canonical mod m[i].
template <bool B60, int K, int S>
__device__ __forceinline__ void garner(const uint64_t (&x)[K], uint64_t (&v)[K], uint32_t k,
                                       const uint64_t* __restrict__ m, const Tw* __restrict__ g) {
  static_assert(K <= S, "register width exceeds the table stride");
#pragma unroll
  for (int i = 0; i < K; ++i) {
    if (i >= (int)k) break;
    const uint64_t mi = m[i], two = mi + mi;
    uint64_t s = 0;
#pragma unroll
    for (int kk = 0; kk < i; ++kk) s = lazy_add<B60>(s, shoup<B60>(v[kk], g[i * S + kk], mi), two);
    // x_i - s + 2 m_i in (0, 3 m_i)
    const uint64_t y = x[i] + two - s;
    v[i] = csub(i == 0 ? x[0] : shoup<B60>(y, g[i * S + i], mi), mi);
  }
}

// sum_i v_i c_i mod p, canonical.  c[i] = prod_{j<i} m_j mod p (Shoup pairs).
template <bool B60, int K>
__device__ __forceinline__ uint64_t mixed_radix_eval(const uint64_t (&v)[K], uint32_t k, const Tw* __restrict__ c,
                                                     uint64_t p) {
  const uint64_t two = p + p;
  uint64_t s = 0;
#pragma unroll
  for (int i = 0; i < K; ++i) {
    if (i >= (int)k) break;
    s = lazy_add<B60>(s, shoup<B60>(v[i], c[i], p), two);
  }
  return csub(s, p);
}

// Below 2^60: sum_i v_i c_i for digits v_i < 2^60 and constants c_i < p stored as
// 30-bit halves.  Each term is four carry-free 32 x 32 + 64-bit multiply-adds into
//   A = sum vl cl,  B = sum (vl ch + vh cl),  C = sum vh ch
// (per term below 2^60, 2^61, 2^60, so eight terms cannot overflow); the exact
// T = A + B 2^30 + C 2^60 < 8 2^60 p < p 2^64 is then Montgomery-reduced once.  The
// constants carry the factor 2^64 that the reduction divides out.  Result canonical.
struct C30 {
  uint32_t l, h;
};
template <int K>
__device__ __forceinline__ uint64_t dot30(const uint32_t (&vl)[K], const uint32_t (&vh)[K], uint32_t k,
                                          const C30* __restrict__ c, uint64_t p, uint64_t ninv) {
  uint64_t r = 0;
#pragma unroll
  for (int i0 = 0; i0 < K; i0 += 8) {
    if (i0 >= (int)k) break;
    uint64_t A = 0, B = 0, C = 0;
#pragma unroll
    for (int i = i0; i < i0 + 8 && i < K; ++i) {
      if (i >= (int)k) break;
      const C30 cc = c[i];
      A += (uint64_t)vl[i] * cc.l;
      B += (uint64_t)vl[i] * cc.h;
      B += (uint64_t)vh[i] * cc.l;
      C += (uint64_t)vh[i] * cc.h;
    }
    const uint64_t blo = B << 30, clo = C << 60;
    Acc128 t;
    t.lo = A + blo;
    t.hi = (B >> 34) + (C >> 4) + (t.lo < blo);
    t.lo += clo;
    t.hi += (t.lo < clo);
    const uint64_t red = csub(redc(t, p, ninv), p);
    r = i0 == 0 ? red : add_mod(r, red, p);
  }
  return r;
}

// Garner digits below 2^60 with each inner sum s_i = sum_{k<i} v_k g_ik as a 30-bit
// half dot product (constants g30[i S + k] = g_ik 2^64 mod m_i, one Montgomery
// reduction), then v_i = (x_i + m_i - s_i) g_ii mod m_i by a Shoup product.  Also
// returns the halves of every digit for the evaluations that follow.
template <int K, int S>
__device__ __forceinline__ void garner30(const uint64_t (&x)[K], uint64_t (&v)[K], uint32_t (&vl)[K],
                                         uint32_t (&vh)[K], uint32_t k, const uint64_t* __restrict__ m,
                                         const uint64_t* __restrict__ ninv, const Tw* __restrict__ g,
                                         const C30* __restrict__ g30) {
  static_assert(K <= S, "register width exceeds the table stride");
#pragma unroll
  for (int i = 0; i < K; ++i) {
    if (i >= (int)k) break;
    uint64_t vi;
    if (i == 0) {
      vi = x[0];
    } else {
      const uint64_t mi = m[i];
      const uint64_t si = dot30<K>(vl, vh, (uint32_t)i, g30 + i * S, mi, ninv[i]);
      vi = csub(shoup<true>(x[i] + mi - si, g[i * S + i], mi), mi);  // x_i + m_i - s_i < 2 m_i
    }
    v[i] = vi;
    vl[i] = (uint32_t)vi & 0x3fffffffu;
    vh[i] = (uint32_t)(vi >> 30);
  }
}

// Coefficient-domain automorphism gather: value of sigma_g(a) at position e.
// i = e * h mod 2n with h = g^-1 mod 2n; sigma_g(a)[e] = a[i] (i < n) or -a[i - n].
struct Gather {
  uint32_t src;
  bool neg;
};
__device__ __forceinline__ Gather gather_index(uint32_t e, uint32_t h, uint32_t logn) {
  const uint32_t n = 1u << logn;
  const uint32_t i = (uint32_t)(((uint64_t)e * h) & (2 * n - 1));
  return Gather{i & (n - 1), i >= n};
}

// Device constants of a key-switch plan (one allocation, offsets in elements).
struct KsDev {
  const uint64_t* moduli;   // [nq + np]
  const Tw* digit_garner;   // [dnum][K][K]   (K = kMaxDigitPrimes)
  const Tw* digit_eval;     // [dnum][nq+np][K]
  const Tw* p_garner;       // [KP][KP]       (KP = kMaxSpecial)
  const Tw* p_eval;         // [nq][KP]
  const Tw* p_inv;          // [nq]
  const uint64_t* p_r64;    // [nq]     P 2^64 mod q_l (hoisted rotations fold P sigma_g(c0) into the key product)
  const Tw* r_scale;        // [nq+np]  2^64 mod q_t
  const C30* digit_eval30;  // [dnum][nq+np][K]  below 2^60: digit products times 2^128 mod q_t
  const C30* p_eval30;      // [nq][KP]           below 2^60: products of P's primes times 2^64
  const C30* digit_garner30;  // [dnum][K][K]     below 2^60: Garner constants times 2^64 (k < i)
  const C30* p_garner30;      // [KP][KP]
  const uint64_t* ninv;     // [nq+np]  -q_t^-1 mod 2^64
};

}  // namespace
}  // namespace nntt
