// Device-side modular arithmetic for gfx950.
//
// Two residue widths share one set of kernels through the traits below:
//   Wide   : q < 2^62, residues in uint64_t.  Lazy (Harvey) butterflies keep
//            values in [0, 4q) < 2^64.  Products by a table constant use Shoup's
//            method with w' = floor(w * 2^64 / q).
//   Narrow : q < 2^30, residues in uint32_t (stored as uint64_t in memory),
//            [0, 4q) < 2^32, Shoup with w' = floor(w * 2^32 / q).
// Products of two variables (pointwise, tensor, key inner product) use Barrett
// reduction of the 128-bit product (see barrett_mul).
//
// CDNA4 issues v_mul_lo_u32 / v_mul_hi_u32 / v_mad_u64_u32 at full rate, so a
// Shoup product is ~16 VALU instructions and a lazy butterfly ~24.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nntt {

// The Shoup remainder y w - Q q, formed mod 2^64 as y w + Q (2^64 - q) from 32-bit
// halves: the two low products in one multiply-add chain (nothing here waits for the
// quotient but the second one), the four cross products only into the high word.
// The empty asm keeps that high word a 32-bit add in place: otherwise the compiler
// re-forms a 64-bit add of a zero-extended value, one more move and add.
__device__ __forceinline__ uint64_t shoup_rem(uint32_t y0, uint32_t y1, uint64_t w, uint64_t Q, uint64_t nq) {
  const uint32_t q0 = (uint32_t)Q, q1 = (uint32_t)(Q >> 32);
  const uint64_t lo = (uint64_t)q0 * (uint32_t)nq + (uint64_t)y0 * (uint32_t)w;
  uint32_t hi = y0 * (uint32_t)(w >> 32) + y1 * (uint32_t)w + q0 * (uint32_t)(nq >> 32) + q1 * (uint32_t)nq;
  hi += (uint32_t)(lo >> 32);
  asm("" : "+v"(hi));
  return ((uint64_t)hi << 32) | (uint32_t)lo;
}

struct Wide {
  using T = uint64_t;
  struct Tw {
    uint64_t w, wp;
  };
  static constexpr int kPadShift = 4;  // one pad slot per 16 elements (128 B of LDS banks)
  static constexpr bool kSignSelect = false;  // values reach 4q < 2^64: full unsigned compare
  static constexpr int kShoupBits = 64;

  // y * w mod q, result in [0, 2q); any y < 2^64.  Q = hi64(y w') >= floor(y w / q) - 1.
  static __device__ __forceinline__ T mul(T y, Tw t, T q) {
    const uint64_t Q = __umul64hi(y, t.wp);
    return shoup_rem((uint32_t)y, (uint32_t)(y >> 32), t.w, Q, 0 - q);
  }
  static __device__ __forceinline__ T load(const uint64_t* p) { return *p; }
  static __device__ __forceinline__ uint64_t widen(T x) { return x; }
};

// q < 2^60: values stay below 4q < 2^62, which allows a Shoup constant scaled by
// 2^62, w' = floor(w * 2^62 / q) < 2^62.  Then with y = y1 2^32 + y0 (y1 < 2^30)
// and w' = p1 2^32 + p0 (p1 < 2^30) the middle sum
//   S = y0 p1 + y1 p0 + hi32(y0 p0) < 2^64
// cannot overflow, and Q = floor(y w' / 2^62) = (y1 p1 2^32 + S) >> 30 (the low
// 32 bits of y0 p0 never change the quotient).  Q >= floor(y w / q) - 1, so the
// remainder stays in [0, 2q).  No carries to track, fewer register-pair moves.
struct Wide60 {
  using T = uint64_t;
  struct Tw {
    uint64_t w, wp;
  };
  static constexpr int kPadShift = 4;
  static constexpr bool kSignSelect = true;  // values < 4q < 2^62
  static constexpr int kShoupBits = 62;

  static __device__ __forceinline__ T mul(T y, Tw t, T q) {
    const uint32_t y0 = (uint32_t)y, y1 = (uint32_t)(y >> 32);
    const uint32_t p0 = (uint32_t)t.wp, p1 = (uint32_t)(t.wp >> 32);
    uint64_t S = (uint64_t)y1 * p0 + __umulhi(y0, p0);
    S = (uint64_t)y0 * p1 + S;
    // (y1 p1 2^32 + S) >> 30 = 4 y1 p1 + (S >> 30): one 64-bit shift and one
    // shift-add.  The empty asm keeps the product whole; otherwise the shift by 2 is
    // folded into p1 and the product splits in two.
    uint64_t P11 = (uint64_t)y1 * p1;
    asm("" : "+v"(P11));
    const uint64_t Q = (P11 << 2) + (S >> 30);
    return shoup_rem(y0, y1, t.w, Q, 0 - q);
  }
  static __device__ __forceinline__ uint64_t widen(T x) { return x; }
};

struct Narrow {
  using T = uint32_t;
  struct Tw {
    uint32_t w, wp;
  };
  static constexpr int kPadShift = 5;  // one pad slot per 32 elements
  static constexpr bool kSignSelect = false;
  static constexpr int kShoupBits = 32;

  static __device__ __forceinline__ T mul(T y, Tw t, T q) {
    uint32_t hi = __umulhi(y, t.wp);
    return y * t.w - hi * q;
  }
  static __device__ __forceinline__ uint64_t widen(T x) { return x; }
};

// x in [0, 2m) -> [0, m)
template <class T>
__device__ __forceinline__ T csub(T x, T m) {
  return x >= m ? x - m : x;
}

// The same for x < 2^63 and m <= 2^62 without compare/carry (no VCC hazards):
// d = x - m is negative exactly when x < m; keep x there, else d.  The select is a
// bit-field insert on the sign mask.
__device__ __forceinline__ uint64_t csub_sign(uint64_t x, uint64_t m) {
  // x + (2^64 - m): a single 64-bit add (v_lshl_add_u64).  The empty asm keeps the
  // optimiser from folding the negation back into a borrow-chain subtraction.
  uint64_t nm = 0 - m;
  asm("" : "+v"(nm));
  const uint64_t d = x + nm;
  const uint32_t mask = (uint32_t)((int32_t)(uint32_t)(d >> 32) >> 31);
  uint32_t lo, hi;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(lo) : "v"(mask), "v"((uint32_t)x), "v"((uint32_t)d));
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(hi) : "v"(mask), "v"((uint32_t)(x >> 32)), "v"((uint32_t)(d >> 32)));
  return ((uint64_t)hi << 32) | lo;
}

// Lazy reduction used by the butterflies (per residue width).
template <class A>
__device__ __forceinline__ typename A::T reduce_once(typename A::T x, typename A::T m) {
  if constexpr (sizeof(typename A::T) == 8 && A::kSignSelect) return csub_sign(x, m);
  else return csub(x, m);
}

// Cooley-Tukey (decimation in time) butterfly with lazy reduction.
// In: x, y in [0, 4q).  Out: x + w y, x - w y + 2q, both in [0, 4q).
// CANON: x is canonical (< q), as on a transform's first stage: no reduction.
template <class A, bool CANON = false>
__device__ __forceinline__ void ct_butterfly(typename A::T& x, typename A::T& y, typename A::Tw w, typename A::T q,
                                             typename A::T two_q) {
  using T = typename A::T;
  T u = CANON ? x : reduce_once<A>(x, two_q);
  T t = A::mul(y, w, q);
  x = u + t;
  y = u - t + two_q;
}

// Gentleman-Sande (decimation in frequency) butterfly with lazy reduction.
// In: x, y in [0, 2q).  Out: x + y, (x - y) w, both in [0, 2q).
// CANON: x, y canonical (< q), as on a transform's first stage: x + y < 2q as it is.
template <class A, bool CANON = false>
__device__ __forceinline__ void gs_butterfly(typename A::T& x, typename A::T& y, typename A::Tw w, typename A::T q,
                                             typename A::T two_q) {
  using T = typename A::T;
  T s = x + y;
  T d = x - y + two_q;
  x = CANON ? s : reduce_once<A>(s, two_q);
  y = A::mul(d, w, q);
}

// The inverse network's last stage with the final n^-1 folded in: (x + y) n^-1 and
// (x - y) w n^-1, each one Shoup product.  In: x, y in [0, 2q).  Out: both in [0, 2q).
template <class A>
__device__ __forceinline__ void gs_butterfly_scaled(typename A::T& x, typename A::T& y, typename A::Tw ninv,
                                                    typename A::Tw wn, typename A::T q, typename A::T two_q) {
  using T = typename A::T;
  const T s = x + y;
  const T d = x - y + two_q;
  x = A::mul(s, ninv, q);
  y = A::mul(d, wn, q);
}

// Barrett reduction of a full product of two canonical 64-bit residues.
// q < 2^62 with k = bitlen(q); mu = floor(2^(2k) / q) < 2^63.
// q1 = floor(x / 2^(k-1)), q3 = floor(q1 * mu / 2^(k+1)); then
// floor(x/q) - 2 <= q3 <= floor(x/q), so x - q3 q lies in [0, 3q).
struct Barrett {
  uint64_t q, mu;
  uint32_t k;
};

__device__ __forceinline__ uint64_t shr128(uint64_t hi, uint64_t lo, uint32_t s) {
  // s in [1, 63]
  return (hi << (64 - s)) | (lo >> s);
}

__device__ __forceinline__ uint64_t barrett_reduce(uint64_t hi, uint64_t lo, const Barrett& b) {
  uint64_t q1 = shr128(hi, lo, b.k - 1);
  uint64_t ph = __umul64hi(q1, b.mu), pl = q1 * b.mu;
  uint64_t q3 = shr128(ph, pl, b.k + 1);
  uint64_t r = lo - q3 * b.q;
  r = csub(r, b.q);
  r = csub(r, b.q);
  return r;
}

__device__ __forceinline__ uint64_t barrett_mul(uint64_t a, uint64_t c, const Barrett& b) {
  return barrett_reduce(__umul64hi(a, c), a * c, b);
}

// The same for q < 2^30 (k <= 30): the product x y < 2^(2k) fits 64 bits, q1 < 2^(k+1)
// and q1 mu < 2^62, so the whole reduction is 64-bit arithmetic of 32-bit operands;
// x y - q3 q lies in [0, 3q) < 2^32.
__device__ __forceinline__ uint32_t barrett_mul_narrow(uint32_t x, uint32_t y, const Barrett& b) {
  const uint64_t p = (uint64_t)x * y;
  const uint64_t q1 = p >> (b.k - 1);
  const uint64_t q3 = (q1 * b.mu) >> (b.k + 1);
  uint32_t r = (uint32_t)(p - q3 * b.q);
  const uint32_t q = (uint32_t)b.q;
  r = csub(r, q);
  return csub(r, q);
}

// Exact 128-bit accumulation of 64 x 64-bit products, and Montgomery reduction with
// R = 2^64: for T = hi 2^64 + lo < q 2^64 and ninv = -q^-1 mod 2^64, m = lo ninv
// makes T + m q divisible by 2^64; the quotient hi + hi64(m q) + [lo != 0] equals
// T 2^-64 mod q and lies in [0, 2q).  (lo + lo64(m q) is 0 or exactly 2^64.)
struct Acc128 {
  uint64_t lo, hi;
};
__device__ __forceinline__ void mac128(Acc128& a, uint64_t x, uint64_t y) {
  const uint64_t lo = x * y;
  a.hi += __umul64hi(x, y);
  a.lo += lo;
  a.hi += (a.lo < lo);
}
__device__ __forceinline__ uint64_t redc(const Acc128& a, uint64_t q, uint64_t ninv) {
  const uint64_t m = a.lo * ninv;
  return a.hi + __umul64hi(m, q) + (a.lo != 0);
}

__device__ __forceinline__ uint64_t add_mod(uint64_t a, uint64_t c, uint64_t q) { return csub(a + c, q); }
__device__ __forceinline__ uint64_t sub_mod(uint64_t a, uint64_t c, uint64_t q) { return a >= c ? a - c : a + q - c; }
__device__ __forceinline__ uint64_t neg_mod(uint64_t a, uint64_t q) { return a ? q - a : 0; }

}  // namespace nntt
