// Negacyclic NTT / inverse NTT kernels for gfx950.
//
// Transform (the library's contract; the pages leave the formula open):
//   forward: ahat[k] = sum_i a[i] psi^((2 brv(k) + 1) i) mod q  (bit-reversed slots)
//   inverse: a[i] = n^-1 sum_k ahat[k] psi^(-(2 brv(k) + 1) i)
// computed in place by the decimation-in-time (Cooley-Tukey) network with the
// psi^brv table, and by the decimation-in-frequency (Gentleman-Sande) network
// with the psi^-brv table.
//
// Stage numbering.  In a transform of size M = 2^m, stage sigma (0 <= sigma < m)
// has 2^sigma butterfly groups at distance M / 2^(sigma+1); the butterfly at
// position j uses table[prefix * 2^sigma + j / (2 * distance)].  A transform of
// size N split into N1 x N2 (row-major, N2 contiguous) runs stages 0..log N1-1
// as N2 independent column transforms (prefix 1) and the remaining stages as N1
// row transforms, row r with prefix N1 + r (the subtree of the bit-reversed
// table rooted at N1 + r).  The same indexing serves both directions; the
// forward network walks sigma upwards, the inverse downwards.
//
// Kernels:
//   ntt_lds_kernel  : whole limb resident in LDS, n <= 2^14 (128 KiB of
//                     residues fit the 160 KiB LDS of one gfx950 workgroup); at
//                     n = 2^14 only for 30-bit residues.
//   ntt_col_kernel / ntt_row_kernel : the two halves for n = 2^15, 2^16, and for
//                     n = 2^14 with 64-bit residues; the intermediate goes through
//                     L2/MALL/HBM between launches.
//   ntt_row_ks_kernel : the key-switch's middle for up to 4 digits -- the forward row
//                     pass of every digit's row tile, the key product of both
//                     components and the inverse row pass, the digits kept in LDS.
//   ntt_row_mac_kernel / ntt_row_mac_hoisted_kernel : the inverse transform's first
//                     (row) pass with the key-switch's key product computed as the
//                     row tile is loaded (more digits, or hoisted rotations whose
//                     digits are gathered through the NTT-domain slot permutation).
//   ct_tensor_coeff_kernel : the coefficient-domain ciphertext product for n <= 2^12,
//                     four forward transforms, slot products and three inverse
//                     transforms of one (ciphertext, limb) in LDS.
// Inside a workgroup, each thread holds one radix-2^r "set" (up to 16 residues)
// in registers and runs r stages on it; sets are exchanged through LDS between
// passes.  LDS rows are padded by one slot per 128 bytes so strided set accesses
// spread over the banks.
#include <algorithm>

#include "ntt_passes.h"

namespace nntt {
namespace {

// The pass machinery (schedules, LDS layout, block placement, passes, finishing)
// is in ntt_passes.h.
// ---------------------------------------------------------------------------
// Whole limb in LDS.
template <int LOGN>
struct LdsCfg {
  static constexpr Sched S = make_sched(LOGN);
  static constexpr int RMAX = S.r[0];
  static constexpr int N = 1 << LOGN;
  static constexpr int NT0 = (N >> RMAX) >= 256 ? (N >> RMAX) : 256;
  static constexpr int NT = NT0 > 1024 ? 1024 : NT0;
  static constexpr int ROWS = (NT << RMAX) / N > 0 ? (NT << RMAX) / N : 1;
};

// GAL: the coefficient-domain automorphism sigma_g is applied while loading
// (residue i of `in` lands, negated when i*g mod 2n >= n, at slot i*g mod n of
// the LDS row), so that the launch computes NTT(sigma_g(in)).  `in` may equal
// `data`: every row is fully loaded before any store.
template <class A, int LOGN, bool FWD, bool GAL>
__global__ __launch_bounds__(LdsCfg<LOGN>::NT) void ntt_lds_kernel(uint64_t* data,
                                                                   const uint64_t* in,
                                                                   const void* __restrict__ tw_all,
                                                                   const ModInfo* __restrict__ mods,
                                                                   uint32_t num_limbs, uint32_t limb_begin,
                                                                   uint64_t total_rows, uint32_t galois) {
  using T = typename A::T;
  using C = LdsCfg<LOGN>;
  constexpr int N = C::N, ROWS = C::ROWS, NT = C::NT;
  constexpr int STRIDE = sub_stride<A>(LOGN);
  __shared__ T lds[ROWS * STRIDE];
  const int tid = threadIdx.x;
  // One row per workgroup: place limb-major across XCDs (see place_block).  Several
  // short rows per workgroup: consecutive rows, so that loads stay coalesced.
  uint64_t row0 = (uint64_t)blockIdx.x * ROWS;
  if (ROWS == 1) row0 = place_block(1, total_rows / num_limbs, num_limbs, 0).row;

  // Coalesced load, two residues per thread per step.  Every load is issued before
  // the first LDS write (a register buffer, no per-row branch), so that their
  // latencies overlap.  A block's rows past the end re-read the last row: their
  // LDS rows are transformed but never stored.
  constexpr int kLoads = (ROWS * N) / (2 * NT);
  static_assert((ROWS * N) % (2 * NT) == 0, "whole iterations");
  ulonglong2 buf[kLoads];
#pragma unroll
  for (int it = 0; it < kLoads; ++it) {
    const int e = 2 * tid + it * 2 * NT;
    const uint64_t r = min(row0 + (uint64_t)(e / N), total_rows - 1);
    buf[it] = *reinterpret_cast<const ulonglong2*>(in + r * N + e % N);
  }
#pragma unroll
  for (int it = 0; it < kLoads; ++it) {
    const int e = 2 * tid + it * 2 * NT;
    const int sub = e / N, pos = e % N;
    const ulonglong2 v = buf[it];
    if (GAL) {
      const uint64_t r = min(row0 + (uint64_t)sub, total_rows - 1);
      const T q = (T)mods[limb_begin + (uint32_t)(r % num_limbs)].q;
      const uint32_t e0 = (uint32_t)(((uint64_t)pos * galois) & (2 * N - 1));
      const uint32_t e1 = (uint32_t)(((uint64_t)(pos + 1) * galois) & (2 * N - 1));
      const T x0 = (T)v.x, x1 = (T)v.y;
      lds[sub * STRIDE + lpos<A>(e0 & (N - 1))] = e0 >= (uint32_t)N ? (x0 ? q - x0 : x0) : x0;
      lds[sub * STRIDE + lpos<A>(e1 & (N - 1))] = e1 >= (uint32_t)N ? (x1 ? q - x1 : x1) : x1;
    } else {
      lds[sub * STRIDE + lpos<A>(pos)] = (T)v.x;
      lds[sub * STRIDE + lpos<A>(pos + 1)] = (T)v.y;
    }
  }
  __syncthreads();

  auto get_sub = [&](int sub) {
    const uint32_t limb = limb_begin + (uint32_t)((row0 + sub) % num_limbs);
    SubParams<A> sp;
    sp.tw = table_of<A>(tw_all, limb, N);
    sp.q = modulus<A>(mods[limb]);
    sp.prefix = 1;
    return sp;
  };
  // Inverse: twiddles on demand (measured on MI355X: n = 2^14, 2048 limbs, 307 -> 291 us;
  // the same at n = 2048).  The n^-1 scaling stays in the store: folded into the last
  // stage as in the column pass it was 1% slower at n = 2^14.
  run_passes<A, FWD, LOGN, ROWS, NT, 0, decltype(get_sub), 0, false, true>(lds, tid, get_sub);

  static_assert((ROWS * N) % (2 * NT) == 0, "whole iterations");
#pragma unroll
  for (int it = 0; it < (ROWS * N) / (2 * NT); ++it) {
    const int e = 2 * tid + it * 2 * NT;
    const int sub = e / N, pos = e % N;
    if (row0 + sub < total_rows) {
      const ModInfo& m = mods[limb_begin + (uint32_t)((row0 + sub) % num_limbs)];
      ulonglong2 v;
      v.x = finish<A, FWD>(lds[sub * STRIDE + lpos<A>(pos)], m);
      v.y = finish<A, FWD>(lds[sub * STRIDE + lpos<A>(pos + 1)], m);
      *reinterpret_cast<ulonglong2*>(data + (row0 + sub) * N + pos) = v;
    }
  }
}

// ---------------------------------------------------------------------------
// Ciphertext product in the coefficient domain, n <= 2^12: one block per (ciphertext,
// limb) holds a0, a1, b0, b1 in LDS, transforms all four, forms
//   d0 = a0 b0,  d1 = a0 b1 + a1 b0,  d2 = a1 b1   (slot by slot, mod q)
// and inverse-transforms the three; only the operands and the result cross HBM.
template <int LOGN>
struct ChainCfg {
  static constexpr Sched S = make_sched(LOGN);
  static constexpr int N = 1 << LOGN;
  static constexpr int NT0 = 4 * (N >> S.r[0]);  // one radix-2^r0 set per thread over four rows
  static constexpr int NT = NT0 < 64 ? 64 : (NT0 > 1024 ? 1024 : NT0);
};
constexpr uint32_t kChainMaxLogN = 12;

template <class A, int LOGN>
__global__ __launch_bounds__(ChainCfg<LOGN>::NT) void ct_tensor_coeff_kernel(
    uint64_t* __restrict__ out, const uint64_t* __restrict__ a, const uint64_t* __restrict__ b,
    const void* __restrict__ tw_fwd, const void* __restrict__ tw_inv, const ModInfo* __restrict__ mods,
    uint32_t num_limbs, uint32_t limb_begin, uint64_t batch) {
  using T = typename A::T;
  constexpr int N = ChainCfg<LOGN>::N, NT = ChainCfg<LOGN>::NT;
  constexpr int STRIDE = sub_stride<A>(LOGN);
  __shared__ T lds[4 * STRIDE];
  const int tid = threadIdx.x;
  const Place pl = place_block(1, batch, num_limbs, 0);
  const uint64_t ct = pl.row / num_limbs;
  const uint32_t l = pl.limb, limb = limb_begin + l;
  const uint64_t plane = (uint64_t)num_limbs * N;
  // row r of the four: a0, a1, b0, b1
  auto src = [&](int r) { return (r < 2 ? a : b) + (2 * ct + (r & 1)) * plane + (uint64_t)l * N; };

  // rows a0, a1, b0, b1, every load issued before the first LDS write
  constexpr int kPairs = 2 * N, kLoads = (kPairs + NT - 1) / NT;
  ulonglong2 buf[kLoads];
#pragma unroll
  for (int it = 0; it < kLoads; ++it) {
    const int e = 2 * (tid + it * NT);
    if (kPairs % NT == 0 || e < 4 * N) buf[it] = *reinterpret_cast<const ulonglong2*>(src(e / N) + e % N);
  }
#pragma unroll
  for (int it = 0; it < kLoads; ++it) {
    const int e = 2 * (tid + it * NT);
    if (kPairs % NT == 0 || e < 4 * N) {
      const int r = e / N, pos = e % N;
      lds[r * STRIDE + lpos<A>(pos)] = (T)buf[it].x;
      lds[r * STRIDE + lpos<A>(pos + 1)] = (T)buf[it].y;
    }
  }
  __syncthreads();

  const ModInfo& m = mods[limb];
  const T q = modulus<A>(m);
  {
    const typename A::Tw* tw = table_of<A>(tw_fwd, limb, N);
    auto get_sub = [&](int) {
      SubParams<A> sp;
      sp.tw = tw;
      sp.q = q;
      sp.prefix = 1;
      return sp;
    };
    run_passes<A, true, LOGN, 4, NT, 0, decltype(get_sub), 0, false, true>(lds, tid, get_sub);
  }
  // d0, d1, d2 over rows 0, 1, 2: each thread reads and writes only its own slots
  const Barrett br = m.br;
  for (int k = tid; k < N; k += NT) {
    const int o = lpos<A>(k);
    const uint64_t x0 = finish<A, true>(lds[o], m), x1 = finish<A, true>(lds[STRIDE + o], m);
    const uint64_t y0 = finish<A, true>(lds[2 * STRIDE + o], m), y1 = finish<A, true>(lds[3 * STRIDE + o], m);
    if constexpr (A::kShoupBits == 32) {  // q < 2^30
      const uint32_t q32 = (uint32_t)br.q;
      lds[o] = barrett_mul_narrow((uint32_t)x0, (uint32_t)y0, br);
      lds[STRIDE + o] = csub(barrett_mul_narrow((uint32_t)x0, (uint32_t)y1, br) +
                                 barrett_mul_narrow((uint32_t)x1, (uint32_t)y0, br), q32);
      lds[2 * STRIDE + o] = barrett_mul_narrow((uint32_t)x1, (uint32_t)y1, br);
    } else {
      lds[o] = (T)barrett_mul(x0, y0, br);
      lds[STRIDE + o] = (T)add_mod(barrett_mul(x0, y1, br), barrett_mul(x1, y0, br), br.q);
      lds[2 * STRIDE + o] = (T)barrett_mul(x1, y1, br);
    }
  }
  __syncthreads();
  {
    const typename A::Tw* tw = table_of<A>(tw_inv, limb, N);
    auto get_sub = [&](int) {
      SubParams<A> sp;
      sp.tw = tw;
      sp.q = q;
      sp.prefix = 1;
      return sp;
    };
    run_passes<A, false, LOGN, 3, NT, 0, decltype(get_sub), 0, false, true>(lds, tid, get_sub);
  }
  constexpr int kOutPairs = 3 * N / 2, kStores = (kOutPairs + NT - 1) / NT;
#pragma unroll
  for (int it = 0; it < kStores; ++it) {
    const int e = 2 * (tid + it * NT);
    if (kOutPairs % NT == 0 || e < 3 * N) {
      const int r = e / N, pos = e % N;
      ulonglong2 v;
      v.x = finish<A, false>(lds[r * STRIDE + lpos<A>(pos)], m);
      v.y = finish<A, false>(lds[r * STRIDE + lpos<A>(pos + 1)], m);
      *reinterpret_cast<ulonglong2*>(out + (3 * ct + r) * plane + (uint64_t)l * N + pos) = v;
    }
  }
}

// Row permutation of the NTT-domain automorphism on an N1 x N2 slot grid.  Slot
// k = r N2 + c evaluates at psi^(2 brv(k) + 1) and 2 brv(k) + 1 mod 2 N1 depends
// on r only, so NTT(sigma_g a)[r N2 + c] = NTT(a)[rp(r) N2 + cp(r, c)] with
//   2 brv(rp) + 1 = g (2 brv(r) + 1)  (mod 2 N1),
//   cp = brv_{log N2}( (g (2 brv(k) + 1) mod 2N) >> (log N1 + 1) ).
template <int LOGB>
__device__ __forceinline__ uint32_t brv_bits(uint32_t x) {
  return __brev(x) >> (32 - LOGB);
}
template <int LOGN1>
__device__ __forceinline__ uint32_t galois_row(uint32_t r, uint32_t g) {
  const uint32_t f = (g * (2 * brv_bits<LOGN1>(r) + 1)) & ((2u << LOGN1) - 1);
  return brv_bits<LOGN1>(f >> 1);
}
template <int LOGN1, int LOGN2>
__device__ __forceinline__ uint32_t galois_col(uint32_t r, uint32_t c, uint32_t g) {
  const uint32_t k = (r << LOGN2) | c;
  const uint32_t f = (uint32_t)(((uint64_t)g * (2 * brv_bits<LOGN1 + LOGN2>(k) + 1)) & ((2u << (LOGN1 + LOGN2)) - 1));
  return brv_bits<LOGN2>(f >> (LOGN1 + 1));
}

// LAST: this launch finishes the transform (canonical output; inverse scaling).
// GAL (forward only): intermediate row rho is written to row slot galois_row(rho, h),
// h = g^-1, i.e. the slot whose source row under g is rho; `in` may equal `data`.
template <class A, int LOGN1, int LOGN2, bool FWD, bool LAST, bool GAL>
__global__ __launch_bounds__(ColCfg<LOGN1>::NT) void ntt_col_kernel(uint64_t* data,
                                                                    const uint64_t* in,
                                                                    const void* __restrict__ tw_all,
                                                                    const ModInfo* __restrict__ mods,
                                                                    uint32_t num_limbs, uint32_t limb_begin,
                                                                    uint64_t batch, uint32_t galois_inv) {
  using T = typename A::T;
  constexpr int N1 = 1 << LOGN1, N2 = 1 << LOGN2, N = N1 * N2;
  constexpr int NT = ColCfg<LOGN1>::NT;
  constexpr int STRIDE = sub_stride<A>(LOGN1);
  constexpr int BLOCKS_PER_LIMB = N2 / kCols;
  __shared__ T lds[kCols * STRIDE];
  const int tid = threadIdx.x;
  const Place pl = place_block(BLOCKS_PER_LIMB, batch, num_limbs, limb_begin);
  const uint64_t row = pl.row;
  const int c0 = (int)pl.tile * kCols;
  const uint32_t limb = pl.limb;
  uint64_t* base = data + row * N + c0;
  const uint64_t* src = in + row * N + c0;

  // Every load of the tile is issued before the first LDS write, so that their
  // latencies overlap.
  constexpr int kLoads = (kCols * N1) / (2 * NT);
  static_assert((kCols * N1) % (2 * NT) == 0, "whole iterations");
  ulonglong2 buf[kLoads];
#pragma unroll
  for (int it = 0; it < kLoads; ++it) {
    const int e = 2 * tid + it * 2 * NT;
    const int rr = e / kCols, c = e % kCols;
    buf[it] = *reinterpret_cast<const ulonglong2*>(src + (size_t)rr * N2 + c);
  }
#pragma unroll
  for (int it = 0; it < kLoads; ++it) {
    const int e = 2 * tid + it * 2 * NT;
    const int rr = e / kCols, c = e % kCols;
    lds[c * STRIDE + lpos<A>(rr)] = (T)buf[it].x;
    lds[(c + 1) * STRIDE + lpos<A>(rr)] = (T)buf[it].y;
  }
  __syncthreads();

  const ModInfo& m = mods[limb];
  SubParams<A> sp;
  sp.tw = table_of<A>(tw_all, limb, N);
  sp.q = modulus<A>(m);
  sp.prefix = 1;
  // The inverse's last launch folds n^-1 into its last stage.
  constexpr bool kFold = !FWD && LAST;
  if constexpr (kFold) scaled_last_stage<A>(m, sp.ninv, sp.w1n);
  auto get_sub = [&](int) { return sp; };
  run_passes<A, FWD, LOGN1, kCols, NT, 0, decltype(get_sub), 1, kFold, FWD>(lds, tid, get_sub);

  static_assert((kCols * N1) % (2 * NT) == 0, "whole iterations");
#pragma unroll
  for (int it = 0; it < (kCols * N1) / (2 * NT); ++it) {
    const int e = 2 * tid + it * 2 * NT;
    const int rr = e / kCols, c = e % kCols;
    ulonglong2 v;
    if (LAST) {
      v.x = finish<A, FWD, kFold>(lds[c * STRIDE + lpos<A>(rr)], m);
      v.y = finish<A, FWD, kFold>(lds[(c + 1) * STRIDE + lpos<A>(rr)], m);
    } else {
      v.x = A::widen(lds[c * STRIDE + lpos<A>(rr)]);
      v.y = A::widen(lds[(c + 1) * STRIDE + lpos<A>(rr)]);
    }
    const uint32_t slot = GAL ? galois_row<LOGN1>((uint32_t)rr, galois_inv) : (uint32_t)rr;
    *reinterpret_cast<ulonglong2*>(base + (size_t)slot * N2 + c) = v;
  }
}

// GAL (forward only): row slot r holds intermediate row galois_row(r, g); the
// output of slot r is that row's transform permuted by galois_col.
template <class A, int LOGN1, int LOGN2, bool FWD, bool LAST, bool GAL>
__global__ __launch_bounds__(RowCfg<LOGN2>::NT) void ntt_row_kernel(uint64_t* __restrict__ data,
                                                                    const void* __restrict__ tw_all,
                                                                    const ModInfo* __restrict__ mods,
                                                                    uint32_t num_limbs, uint32_t limb_begin,
                                                                    uint64_t batch, uint32_t galois) {
  using T = typename A::T;
  constexpr int N1 = 1 << LOGN1, N2 = 1 << LOGN2, N = N1 * N2;
  constexpr int NT = RowCfg<LOGN2>::NT;
  constexpr int STRIDE = sub_stride<A>(LOGN2);
  constexpr int BLOCKS_PER_LIMB = N1 / kRows;
  __shared__ T lds[kRows * STRIDE];
  const int tid = threadIdx.x;
  const Place pl = place_block(BLOCKS_PER_LIMB, batch, num_limbs, limb_begin);
  const uint64_t row = pl.row;
  const int r0 = (int)pl.tile * kRows;
  const uint32_t limb = pl.limb;
  uint64_t* base = data + row * N + (size_t)r0 * N2;

  constexpr int kLoads = (kRows * N2) / (2 * NT);
  static_assert((kRows * N2) % (2 * NT) == 0, "whole iterations");
  ulonglong2 buf[kLoads];
#pragma unroll
  for (int it = 0; it < kLoads; ++it) buf[it] = *reinterpret_cast<const ulonglong2*>(base + 2 * tid + it * 2 * NT);
#pragma unroll
  for (int it = 0; it < kLoads; ++it) {
    const int e = 2 * tid + it * 2 * NT;
    const int sub = e / N2, pos = e % N2;
    lds[sub * STRIDE + lpos<A>(pos)] = (T)buf[it].x;
    lds[sub * STRIDE + lpos<A>(pos + 1)] = (T)buf[it].y;
  }
  __syncthreads();

  const ModInfo& m = mods[limb];
  const typename A::Tw* tw = table_of<A>(tw_all, limb, N);
  const T q = modulus<A>(m);
  auto get_sub = [&](int sub) {
    SubParams<A> sp;
    sp.tw = tw;
    sp.q = q;
    sp.prefix = (uint32_t)N1 + (GAL ? galois_row<LOGN1>((uint32_t)(r0 + sub), galois) : (uint32_t)(r0 + sub));
    return sp;
  };
  constexpr bool kRowT = LOGN2 == (int)kPermRowLog && row_tw_permuted(LOGN1 + LOGN2);
  run_passes<A, FWD, LOGN2, kRows, NT, 0, decltype(get_sub), 1, false, !FWD, kRowT>(lds, tid, get_sub);

  static_assert((kRows * N2) % (2 * NT) == 0, "whole iterations");
#pragma unroll
  for (int it = 0; it < (kRows * N2) / (2 * NT); ++it) {
    const int e = 2 * tid + it * 2 * NT;
    const int sub = e / N2, pos = e % N2;
    ulonglong2 v;
    if (GAL) {
      const uint32_t r = (uint32_t)(r0 + sub);
      const int p0 = (int)galois_col<LOGN1, LOGN2>(r, (uint32_t)pos, galois);
      const int p1 = (int)galois_col<LOGN1, LOGN2>(r, (uint32_t)pos + 1, galois);
      v.x = finish<A, FWD>(lds[sub * STRIDE + lpos<A>(p0)], m);
      v.y = finish<A, FWD>(lds[sub * STRIDE + lpos<A>(p1)], m);
    } else if (LAST) {
      v.x = finish<A, FWD>(lds[sub * STRIDE + lpos<A>(pos)], m);
      v.y = finish<A, FWD>(lds[sub * STRIDE + lpos<A>(pos + 1)], m);
    } else {
      v.x = A::widen(lds[sub * STRIDE + lpos<A>(pos)]);
      v.y = A::widen(lds[sub * STRIDE + lpos<A>(pos + 1)]);
    }
    *reinterpret_cast<ulonglong2*>(base + e) = v;
  }
}

// The key product of the key-switch fused into the inverse transform's first (row)
// pass.  Tensor row poly * nqp + t of the accumulator, poly = 2 b + c, is
//   acc = sum_j ext[b][j][t] * ksk[j][c][t]   (mod q_t)
// computed as it is loaded: the digits are in Montgomery form (times 2^64), so the
// exact 128-bit sum of up to `chunk` products is reduced once per chunk.  The rest is
// the ordinary Gentleman-Sande row pass; the column pass follows unchanged.
struct MacSrc {
  const uint64_t* ext;  // [batch][dnum][nqp][n]
  const uint64_t* ksk;  // [dnum][2][nqp][n]
  uint32_t dnum, chunk;
  // Hoisted rotations only (nullptr otherwise): NTT(c0) [batch][nq][n] and, per prime of
  // Q, P 2^64 mod q.  Component 0 of every Q prime then also sums P * NTT(c0) at the
  // rotation's slots, i.e. P sigma_g(c0) in the NTT domain, so that ModDown yields
  // sigma_g(c0) + ModDown(acc_0) with no additive input (floor((X + P Y) / P) equals
  // floor(X / P) + Y for every integer Y, and Q vanishes modulo each q).
  const uint64_t* c0hat;
  const uint64_t* pr64;
  uint32_t nq;
};

// Key residues are read once per launch: non-temporal loads keep them from evicting
// the digits, which the hoisted product reads once per rotation and component.
__device__ __forceinline__ ulonglong2 load_key(const uint64_t* p) { return load_tile<true>(p); }

// DN > 0: dnum == DN and DN products fit one reduction (all loads of an element pair
// are issued before any arithmetic); DN == 0: any dnum, chunked reductions.
template <class A, int LOGN1, int LOGN2, int DN>
__global__ __launch_bounds__(RowCfg<LOGN2>::NT) void ntt_row_mac_kernel(uint64_t* __restrict__ acc, MacSrc ms,
                                                                        const void* __restrict__ tw_all,
                                                                        const ModInfo* __restrict__ mods,
                                                                        uint32_t nqp, uint64_t polys) {
  using T = typename A::T;
  constexpr int N1 = 1 << LOGN1, N2 = 1 << LOGN2, N = N1 * N2;
  constexpr int NT = RowCfg<LOGN2>::NT;
  constexpr int STRIDE = sub_stride<A>(LOGN2);
  constexpr int BLOCKS_PER_LIMB = N1 / kRows;
  __shared__ T lds[kRows * STRIDE];
  const int tid = threadIdx.x;
  const Place pl = place_block(BLOCKS_PER_LIMB, polys, nqp, 0);
  const uint64_t row = pl.row, poly = row / nqp;
  const uint32_t t = pl.limb;
  const size_t off = (size_t)pl.tile * kRows * N2;  // first element of this tile in the limb
  const uint64_t plane = (uint64_t)nqp * N;
  const uint64_t* xe = ms.ext + ((poly >> 1) * ms.dnum * nqp + t) * (uint64_t)N + off;
  const uint64_t* kk = ms.ksk + ((poly & 1) * nqp + t) * (uint64_t)N + off;
  const ModInfo& m = mods[t];
  const uint64_t q = m.q, ninv = m.mont_ninv;

  constexpr int kIters = (kRows * N2) / (2 * NT);
  static_assert((kRows * N2) % (2 * NT) == 0, "whole iterations");
#pragma unroll 2
  for (int it = 0; it < kIters; ++it) {
    const int e = 2 * tid + it * 2 * NT;
    Acc128 a0{0, 0}, a1{0, 0};
    uint64_t r0 = 0, r1 = 0;
    if constexpr (DN > 0) {
      ulonglong2 d[DN], k[DN];
#pragma unroll
      for (int j = 0; j < DN; ++j) {
        d[j] = *reinterpret_cast<const ulonglong2*>(xe + j * plane + e);
        k[j] = load_key(kk + 2 * j * plane + e);
      }
#pragma unroll
      for (int j = 0; j < DN; ++j) {
        mac128(a0, d[j].x, k[j].x);
        mac128(a1, d[j].y, k[j].y);
      }
      r0 = csub(redc(a0, q, ninv), q);
      r1 = csub(redc(a1, q, ninv), q);
    } else {
    uint32_t c = 0;
    for (uint32_t j = 0; j < ms.dnum; ++j) {
      const ulonglong2 d = *reinterpret_cast<const ulonglong2*>(xe + j * plane + e);
      const ulonglong2 k = load_key(kk + 2 * j * plane + e);
      mac128(a0, d.x, k.x);
      mac128(a1, d.y, k.y);
      if (++c == ms.chunk || j + 1 == ms.dnum) {
        r0 = add_mod(r0, csub(redc(a0, q, ninv), q), q);
        r1 = add_mod(r1, csub(redc(a1, q, ninv), q), q);
        a0 = Acc128{0, 0};
        a1 = Acc128{0, 0};
        c = 0;
      }
    }
    }
    const int sub = e / N2, pos = e % N2;
    lds[sub * STRIDE + lpos<A>(pos)] = (T)r0;
    lds[sub * STRIDE + lpos<A>(pos + 1)] = (T)r1;
  }
  __syncthreads();

  const typename A::Tw* tw = table_of<A>(tw_all, t, N);
  const T qt = modulus<A>(m);
  auto get_sub = [&](int sub) {
    SubParams<A> sp;
    sp.tw = tw;
    sp.q = qt;
    sp.prefix = (uint32_t)N1 + (uint32_t)(pl.tile * kRows + sub);
    return sp;
  };
  run_passes<A, false, LOGN2, kRows, NT, 0, decltype(get_sub), -1, false, true,
             LOGN2 == (int)kPermRowLog && row_tw_permuted(LOGN1 + LOGN2)>(lds, tid, get_sub);

  uint64_t* base = acc + row * N + off;
  static_assert((kRows * N2) % (2 * NT) == 0, "whole iterations");
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int e = 2 * tid + it * 2 * NT;
    const int sub = e / N2, pos = e % N2;
    ulonglong2 v;
    v.x = A::widen(lds[sub * STRIDE + lpos<A>(pos)]);
    v.y = A::widen(lds[sub * STRIDE + lpos<A>(pos + 1)]);
    *reinterpret_cast<ulonglong2*>(base + e) = v;
  }
}

// The middle of a key-switch for n = N1 x 2^8 in one block per (ciphertext b, limb t,
// tile of ROWS rows): the forward transform's row pass of every digit's tile (the digits
// come from the forward column pass, [batch][DN][nqp][n]), the key product of both
// components,
//   acc_c = sum_j NTT(ext_j)[t] * ksk[j][c][t]   (mod q_t),
// and the inverse transform's row pass of both accumulators, which are stored as the
// intermediate of the inverse ([batch][2][nqp][n]) for its column pass.  The
// NTT-domain digits never leave LDS.  The digits carry the factor 2^64 of ModUp's
// Montgomery form, so the exact 128-bit sum of the DN products (DN q^2 < q 2^64 for
// DN <= 4 and q < 2^62) is reduced once by Montgomery to the plain residue.
template <int DN>
constexpr int ks_tiles() {
  return DN > 2 ? DN : 2;  // LDS tiles: the DN digit tiles, reused for the two accumulators
}
template <int DN, int ROWS>
constexpr int ks_threads() {
  return 16 * ROWS * ks_tiles<DN>();  // one radix-16 set of a 2^8 row per thread and pass
}

template <class A, int LOGN1, int DN, int ROWS>
__global__ __launch_bounds__((ks_threads<DN, ROWS>())) void ntt_row_ks_kernel(
    uint64_t* __restrict__ acc, const uint64_t* __restrict__ ext, const uint64_t* __restrict__ ksk,
    const void* __restrict__ tw_fwd, const void* __restrict__ tw_inv, const ModInfo* __restrict__ mods, uint32_t nqp,
    uint64_t batch) {
  using T = typename A::T;
  constexpr int LOGN2 = 8;
  constexpr int N1 = 1 << LOGN1, N2 = 1 << LOGN2, N = N1 * N2;
  constexpr int TILES = ks_tiles<DN>(), NT = ks_threads<DN, ROWS>();
  constexpr int STRIDE = sub_stride<A>(LOGN2);
  constexpr int TILE = ROWS * N2;  // residues of one tile
  __shared__ T lds[TILES * ROWS * STRIDE];
  const int tid = threadIdx.x;
  const Place pl = place_block(N1 / ROWS, batch, nqp, 0);
  const uint64_t b = pl.row / nqp;
  const uint32_t t = pl.limb;
  const int r0 = (int)pl.tile * ROWS;
  const size_t off = (size_t)r0 * N2;  // first element of the tile in the limb
  const uint64_t plane = (uint64_t)nqp * N;
  const uint64_t* xe = ext + (b * DN * nqp + t) * (uint64_t)N + off;  // digit j at + j plane
  const uint64_t* kk = ksk + (uint64_t)t * N + off;                   // key (j, c) at + (2 j + c) plane
  uint64_t* ao = acc + (b * 2 * nqp + t) * (uint64_t)N + off;          // component c at + c plane

  // Digit tiles, every load issued before the first LDS write.
  constexpr int kLoads = (DN * TILE + 2 * NT - 1) / (2 * NT);
  ulonglong2 buf[kLoads];
#pragma unroll
  for (int it = 0; it < kLoads; ++it) {
    const int e = 2 * tid + it * 2 * NT;
    if (e < DN * TILE) buf[it] = *reinterpret_cast<const ulonglong2*>(xe + (e / TILE) * plane + e % TILE);
  }
#pragma unroll
  for (int it = 0; it < kLoads; ++it) {
    const int e = 2 * tid + it * 2 * NT;
    if (e < DN * TILE) {
      const int sub = e / N2, pos = e % N2;  // sub = j ROWS + row within the tile
      lds[sub * STRIDE + lpos<A>(pos)] = (T)buf[it].x;
      lds[sub * STRIDE + lpos<A>(pos + 1)] = (T)buf[it].y;
    }
  }
  __syncthreads();

  const ModInfo& m = mods[t];
  const T qt = modulus<A>(m);
  constexpr bool kPerm = row_tw_permuted(LOGN1 + LOGN2);
  {
    const typename A::Tw* tw = table_of<A>(tw_fwd, t, N);
    auto get_sub = [&](int sub) {
      SubParams<A> sp;
      sp.tw = tw;
      sp.q = qt;
      sp.prefix = (uint32_t)N1 + (uint32_t)(r0 + sub % ROWS);
      return sp;
    };
    run_passes<A, true, LOGN2, DN * ROWS, NT, 0, decltype(get_sub), 1, false, false, kPerm>(lds, tid, get_sub);
  }

  // Key product: each thread reads its own element pairs of every digit tile and writes
  // the two accumulators to the same positions of tiles 0 and 1 (no other thread
  // touches those positions, so no barrier is needed between the reads and writes).
  const uint64_t q = m.q, ninv = m.mont_ninv;
#pragma unroll 2
  for (int p = tid; p < TILE / 2; p += NT) {
    const int e = 2 * p;
    const int row = e / N2, pos = e % N2;
    ulonglong2 k0[DN], k1[DN];
#pragma unroll
    for (int j = 0; j < DN; ++j) {
      k0[j] = load_key(kk + (2 * j) * plane + e);
      k1[j] = load_key(kk + (2 * j + 1) * plane + e);
    }
    Acc128 s0x{0, 0}, s0y{0, 0}, s1x{0, 0}, s1y{0, 0};
#pragma unroll
    for (int j = 0; j < DN; ++j) {
      T* d = lds + (j * ROWS + row) * STRIDE;
      const uint64_t dx = finish<A, true>(d[lpos<A>(pos)], m);  // canonical NTT-domain digit
      const uint64_t dy = finish<A, true>(d[lpos<A>(pos + 1)], m);
      mac128(s0x, dx, k0[j].x);
      mac128(s0y, dy, k0[j].y);
      mac128(s1x, dx, k1[j].x);
      mac128(s1y, dy, k1[j].y);
    }
    T* a0 = lds + row * STRIDE;
    T* a1 = lds + (ROWS + row) * STRIDE;
    a0[lpos<A>(pos)] = (T)csub(redc(s0x, q, ninv), q);
    a0[lpos<A>(pos + 1)] = (T)csub(redc(s0y, q, ninv), q);
    a1[lpos<A>(pos)] = (T)csub(redc(s1x, q, ninv), q);
    a1[lpos<A>(pos + 1)] = (T)csub(redc(s1y, q, ninv), q);
  }
  __syncthreads();

  {
    const typename A::Tw* tw = table_of<A>(tw_inv, t, N);
    auto get_sub = [&](int sub) {
      SubParams<A> sp;
      sp.tw = tw;
      sp.q = qt;
      sp.prefix = (uint32_t)N1 + (uint32_t)(r0 + sub % ROWS);
      return sp;
    };
    run_passes<A, false, LOGN2, 2 * ROWS, NT, 0, decltype(get_sub), -1, false, true, kPerm>(lds, tid, get_sub);
  }

  // Both accumulator tiles, unreduced (the inverse column pass finishes them).
  constexpr int kStores = (2 * TILE + 2 * NT - 1) / (2 * NT);
#pragma unroll
  for (int it = 0; it < kStores; ++it) {
    const int e = 2 * tid + it * 2 * NT;
    if (e < 2 * TILE) {
      const int sub = e / N2, pos = e % N2;  // sub = c ROWS + row
      ulonglong2 v;
      v.x = A::widen(lds[sub * STRIDE + lpos<A>(pos)]);
      v.y = A::widen(lds[sub * STRIDE + lpos<A>(pos + 1)]);
      *reinterpret_cast<ulonglong2*>(ao + (e / TILE) * plane + e % TILE) = v;
    }
  }
}

// Hoisted rotations: accumulator row poly * nqp + t, poly = (r * batch + b) * 2 + c, is
//   sum_j ext[b][j][t][slot_{g_r}(k)] * ksk[r][j][c][t][k]   (mod q_t)
// for each slot k of the row tile.  A row tile is an aligned segment of slots, so the
// slots it gathers form one aligned segment of each digit (see ntt_slot).
template <class A, int LOGN1, int LOGN2, int DN>
__global__ __launch_bounds__(RowCfg<LOGN2>::NT) void ntt_row_mac_hoisted_kernel(
    uint64_t* __restrict__ acc, MacSrc ms, const void* __restrict__ tw_all, const ModInfo* __restrict__ mods,
    uint32_t nqp, uint64_t polys, uint32_t batch, HoistArgs ha) {
  using T = typename A::T;
  constexpr int N1 = 1 << LOGN1, N2 = 1 << LOGN2, N = N1 * N2;
  constexpr int NT = RowCfg<LOGN2>::NT;
  constexpr int STRIDE = sub_stride<A>(LOGN2);
  constexpr int BLOCKS_PER_LIMB = N1 / kRows;
  __shared__ T lds[kRows * STRIDE];
  const int tid = threadIdx.x;
  const Place pl = place_block(BLOCKS_PER_LIMB, polys, nqp, 0);
  const uint64_t row = pl.row, poly = row / nqp, rb = poly >> 1;
  const uint32_t t = pl.limb, rot = (uint32_t)(rb / batch), g = ha.g[rot];
  const uint64_t b = rb % batch;
  const size_t off = (size_t)pl.tile * kRows * N2;
  const uint64_t plane = (uint64_t)nqp * N;
  const uint64_t* xe = ms.ext + (b * ms.dnum * nqp + t) * (uint64_t)N;
  const uint64_t* kk = ms.ksk + (((uint64_t)rot * ms.dnum * 2 + (poly & 1)) * nqp + t) * (uint64_t)N + off;
  const ModInfo& m = mods[t];
  const uint64_t q = m.q, ninv = m.mont_ninv;
  const bool fold = DN > 0 && ms.c0hat != nullptr && (poly & 1) == 0 && t < ms.nq;
  const uint64_t* cz = fold ? ms.c0hat + (b * ms.nq + t) * (uint64_t)N : nullptr;
  const uint64_t pr = fold ? ms.pr64[t] : 0;

  constexpr int kIters = (kRows * N2) / (2 * NT);
  static_assert((kRows * N2) % (2 * NT) == 0, "whole iterations");
#pragma unroll 2
  for (int it = 0; it < kIters; ++it) {
    const int e = 2 * tid + it * 2 * NT;
    const uint32_t k0 = (uint32_t)(off + e);
    const uint32_t s0 = ntt_slot(k0, g, LOGN1 + LOGN2), s1 = ntt_slot(k0 + 1, g, LOGN1 + LOGN2);
    Acc128 a0{0, 0}, a1{0, 0};
    uint64_t r0 = 0, r1 = 0;
    if constexpr (DN > 0) {
      uint64_t d0[DN], d1[DN];
      ulonglong2 k[DN];
#pragma unroll
      for (int j = 0; j < DN; ++j) {
        d0[j] = xe[j * plane + s0];
        d1[j] = xe[j * plane + s1];
        k[j] = load_key(kk + 2 * j * plane + e);
      }
      uint64_t z0 = 0, z1 = 0;
      if (fold) {
        z0 = cz[s0];
        z1 = cz[s1];
      }
#pragma unroll
      for (int j = 0; j < DN; ++j) {
        mac128(a0, d0[j], k[j].x);
        mac128(a1, d1[j], k[j].y);
      }
      if (fold) {  // DN + 1 products: the launcher checks (DN + 1) q < 2^64
        mac128(a0, z0, pr);
        mac128(a1, z1, pr);
      }
      r0 = csub(redc(a0, q, ninv), q);
      r1 = csub(redc(a1, q, ninv), q);
    } else {
      uint32_t c = 0;
      for (uint32_t j = 0; j < ms.dnum; ++j) {
        const ulonglong2 k = load_key(kk + 2 * j * plane + e);
        mac128(a0, xe[j * plane + s0], k.x);
        mac128(a1, xe[j * plane + s1], k.y);
        if (++c == ms.chunk || j + 1 == ms.dnum) {
          r0 = add_mod(r0, csub(redc(a0, q, ninv), q), q);
          r1 = add_mod(r1, csub(redc(a1, q, ninv), q), q);
          a0 = Acc128{0, 0};
          a1 = Acc128{0, 0};
          c = 0;
        }
      }
    }
    const int sub = e / N2, pos = e % N2;
    lds[sub * STRIDE + lpos<A>(pos)] = (T)r0;
    lds[sub * STRIDE + lpos<A>(pos + 1)] = (T)r1;
  }
  __syncthreads();

  const typename A::Tw* tw = table_of<A>(tw_all, t, N);
  const T qt = modulus<A>(m);
  auto get_sub = [&](int sub) {
    SubParams<A> sp;
    sp.tw = tw;
    sp.q = qt;
    sp.prefix = (uint32_t)N1 + (uint32_t)(pl.tile * kRows + sub);
    return sp;
  };
  run_passes<A, false, LOGN2, kRows, NT, 0, decltype(get_sub), -1, false, true,
             LOGN2 == (int)kPermRowLog && row_tw_permuted(LOGN1 + LOGN2)>(lds, tid, get_sub);

  uint64_t* base = acc + row * N + off;
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int e = 2 * tid + it * 2 * NT;
    const int sub = e / N2, pos = e % N2;
    ulonglong2 v;
    v.x = A::widen(lds[sub * STRIDE + lpos<A>(pos)]);
    v.y = A::widen(lds[sub * STRIDE + lpos<A>(pos + 1)]);
    *reinterpret_cast<ulonglong2*>(base + e) = v;
  }
}

// ---------------------------------------------------------------------------
// What one launch sequence computes.
enum class Op { kForward, kInverse, kForwardGalois };

template <class A>
const void* tables_for(const ntt_plan* p, Op op) {
  const bool inv = op == Op::kInverse;
  if (A::kShoupBits == 64) return inv ? (const void*)p->d_inv : (const void*)p->d_fwd;
  if (A::kShoupBits == 62) return inv ? (const void*)p->d_inv60 : (const void*)p->d_fwd60;
  return inv ? (const void*)p->d_inv32 : (const void*)p->d_fwd32;
}

template <class A, int LOGN>
hipError_t launch_lds(const ntt_plan* p, uint64_t* data, const uint64_t* in, uint64_t rows, uint32_t limb_begin,
                      uint32_t num_limbs, Op op, uint32_t g, hipStream_t s) {
  using C = LdsCfg<LOGN>;
  const void* tw = tables_for<A>(p, op);
  const uint64_t blocks = (rows + C::ROWS - 1) / C::ROWS;
  const dim3 grid((uint32_t)blocks), block(C::NT);
  if (op == Op::kInverse)
    hipLaunchKernelGGL((ntt_lds_kernel<A, LOGN, false, false>), grid, block, 0, s, data, in, tw, p->d_mods,
                       num_limbs, limb_begin, rows, 1u);
  else if (op == Op::kForward)
    hipLaunchKernelGGL((ntt_lds_kernel<A, LOGN, true, false>), grid, block, 0, s, data, in, tw, p->d_mods,
                       num_limbs, limb_begin, rows, 1u);
  else
    hipLaunchKernelGGL((ntt_lds_kernel<A, LOGN, true, true>), grid, block, 0, s, data, in, tw, p->d_mods,
                       num_limbs, limb_begin, rows, g);
  return hipGetLastError();
}

template <class A, int LOGN1, int LOGN2>
hipError_t launch_split(const ntt_plan* p, uint64_t* data, const uint64_t* in, uint64_t rows, uint32_t limb_begin,
                        uint32_t num_limbs, Op op, uint32_t g, hipStream_t s) {
  const void* tw = tables_for<A>(p, op);
  const uint64_t batch = rows / num_limbs;
  const dim3 col_grid((uint32_t)(rows * ((1u << LOGN2) / kCols))), col_block(ColCfg<LOGN1>::NT);
  const dim3 row_grid((uint32_t)(rows * ((1u << LOGN1) / kRows))), row_block(RowCfg<LOGN2>::NT);
  if (op == Op::kForward) {
    hipLaunchKernelGGL((ntt_col_kernel<A, LOGN1, LOGN2, true, false, false>), col_grid, col_block, 0, s, data, in,
                       tw, p->d_mods, num_limbs, limb_begin, batch, 1u);
    hipLaunchKernelGGL((ntt_row_kernel<A, LOGN1, LOGN2, true, true, false>), row_grid, row_block, 0, s, data, tw,
                       p->d_mods, num_limbs, limb_begin, batch, 1u);
  } else if (op == Op::kForwardGalois) {
    const uint32_t two_n = 2u << (LOGN1 + LOGN2);
    const uint32_t h = (uint32_t)host_invmod(g % two_n, two_n);
    hipLaunchKernelGGL((ntt_col_kernel<A, LOGN1, LOGN2, true, false, true>), col_grid, col_block, 0, s, data, in,
                       tw, p->d_mods, num_limbs, limb_begin, batch, h);
    hipLaunchKernelGGL((ntt_row_kernel<A, LOGN1, LOGN2, true, true, true>), row_grid, row_block, 0, s, data, tw,
                       p->d_mods, num_limbs, limb_begin, batch, g);
  } else {
    hipLaunchKernelGGL((ntt_row_kernel<A, LOGN1, LOGN2, false, false, false>), row_grid, row_block, 0, s, data, tw,
                       p->d_mods, num_limbs, limb_begin, batch, 1u);
    hipLaunchKernelGGL((ntt_col_kernel<A, LOGN1, LOGN2, false, true, false>), col_grid, col_block, 0, s, data, data,
                       tw, p->d_mods, num_limbs, limb_begin, batch, 1u);
  }
  return hipGetLastError();
}

template <class A, int LOGN1, int LOGN2>
hipError_t launch_mac_split(const ntt_plan* p, uint64_t* acc, const MacSrc& ms, uint64_t batch, uint32_t nqp,
                            hipStream_t s) {
  const void* tw = tables_for<A>(p, Op::kInverse);
  const uint64_t polys = 2 * batch, rows = polys * nqp;
  const dim3 col_grid((uint32_t)(rows * ((1u << LOGN2) / kCols))), col_block(ColCfg<LOGN1>::NT);
  const dim3 row_grid((uint32_t)(rows * ((1u << LOGN1) / kRows))), row_block(RowCfg<LOGN2>::NT);
  const bool one = ms.dnum <= ms.chunk;  // a single reduction covers every digit
#define NNTT_MAC_ROW(D) \
  hipLaunchKernelGGL((ntt_row_mac_kernel<A, LOGN1, LOGN2, D>), row_grid, row_block, 0, s, acc, ms, tw, p->d_mods, nqp, polys)
  if (one && ms.dnum == 1) NNTT_MAC_ROW(1);
  else if (one && ms.dnum == 2) NNTT_MAC_ROW(2);
  else if (one && ms.dnum == 3) NNTT_MAC_ROW(3);
  else if (one && ms.dnum == 4) NNTT_MAC_ROW(4);
  else NNTT_MAC_ROW(0);
#undef NNTT_MAC_ROW
  hipLaunchKernelGGL((ntt_col_kernel<A, LOGN1, LOGN2, false, true, false>), col_grid, col_block, 0, s, acc, acc, tw,
                     p->d_mods, nqp, 0u, polys, 1u);
  return hipGetLastError();
}

template <class A, int LOGN1, int LOGN2>
hipError_t launch_mac_hoisted_split(const ntt_plan* p, uint64_t* acc, const MacSrc& ms, uint64_t batch,
                                    uint32_t num_rot, uint32_t nqp, const HoistArgs& ha, hipStream_t s) {
  const void* tw = tables_for<A>(p, Op::kInverse);
  const uint64_t polys = 2 * batch * num_rot, rows = polys * nqp;
  const dim3 col_grid((uint32_t)(rows * ((1u << LOGN2) / kCols))), col_block(ColCfg<LOGN1>::NT);
  const dim3 row_grid((uint32_t)(rows * ((1u << LOGN1) / kRows))), row_block(RowCfg<LOGN2>::NT);
  const bool one = ms.dnum <= ms.chunk;
#define NNTT_MAC_ROW(D)                                                                                      \
  hipLaunchKernelGGL((ntt_row_mac_hoisted_kernel<A, LOGN1, LOGN2, D>), row_grid, row_block, 0, s, acc, ms, tw, \
                     p->d_mods, nqp, polys, (uint32_t)batch, ha)
  if (one && ms.dnum == 1) NNTT_MAC_ROW(1);
  else if (one && ms.dnum == 2) NNTT_MAC_ROW(2);
  else if (one && ms.dnum == 3) NNTT_MAC_ROW(3);
  else if (one && ms.dnum == 4) NNTT_MAC_ROW(4);
  else NNTT_MAC_ROW(0);
#undef NNTT_MAC_ROW
  hipLaunchKernelGGL((ntt_col_kernel<A, LOGN1, LOGN2, false, true, false>), col_grid, col_block, 0, s, acc, acc, tw,
                     p->d_mods, nqp, 0u, polys, 1u);
  return hipGetLastError();
}

template <class A>
hipError_t launch_mac_hoisted_any(const ntt_plan* p, uint64_t* acc, const MacSrc& ms, uint64_t batch,
                                  uint32_t num_rot, uint32_t nqp, const HoistArgs& ha, hipStream_t s) {
  if (p->logn == 15) return launch_mac_hoisted_split<A, 7, 8>(p, acc, ms, batch, num_rot, nqp, ha, s);
  if (p->logn == 16) return launch_mac_hoisted_split<A, 8, 8>(p, acc, ms, batch, num_rot, nqp, ha, s);
  return hipErrorNotSupported;
}

template <class A>
hipError_t launch_mac_any(const ntt_plan* p, uint64_t* acc, const MacSrc& ms, uint64_t batch, uint32_t nqp,
                          hipStream_t s) {
  if (p->logn == 15) return launch_mac_split<A, 7, 8>(p, acc, ms, batch, nqp, s);
  if (p->logn == 16) return launch_mac_split<A, 8, 8>(p, acc, ms, batch, nqp, s);
  return hipErrorNotSupported;
}

// The middle of a key-switch for the two-pass sizes: the forward column pass over the
// digits ext [batch][DN][nqp][n] (in place), ntt_row_ks_kernel into acc
// [batch][2][nqp][n], and the inverse column pass over acc.  Batches go in parts that
// keep each launch within the launch cap.
// Rows per fused tile, measured on MI355X (one key-switch at n = 2^16, 24 + 8 primes,
// 3 digits): 4 rows 200 us, 8 rows 207-212 us; on-demand twiddles instead of requesting
// a set's twiddles up front: 208 and 211 us.
constexpr int kKsRows = 4;
template <class A, int LOGN1, int DN>
hipError_t launch_ks_middle_split(const ntt_plan* p, uint64_t* acc, uint64_t* ext, const uint64_t* ksk,
                                  uint64_t batch, uint32_t nqp, hipStream_t s) {
  constexpr int LOGN2 = 8;
  constexpr uint32_t kColBlocks = (1u << LOGN2) / kCols, kRowBlocks = (1u << LOGN1) / kKsRows;
  constexpr uint32_t kColNT = ColCfg<LOGN1>::NT, kKsNT = ks_threads<DN, kKsRows>();
  const void* twf = tables_for<A>(p, Op::kForward);
  const void* twi = tables_for<A>(p, Op::kInverse);
  const uint64_t N = 1ull << (LOGN1 + LOGN2);
  const uint64_t per_ct = std::max<uint64_t>({(uint64_t)DN * nqp * kColBlocks * kColNT,
                                              (uint64_t)nqp * kRowBlocks * kKsNT,
                                              2ull * nqp * kColBlocks * kColNT});
  const uint64_t per = items_per_launch(per_ct);
  if (per == 0) return hipErrorNotSupported;
  for (uint64_t b0 = 0; b0 < batch; b0 += per) {
    const uint64_t nb = std::min(per, batch - b0);
    uint64_t* e = ext + b0 * DN * nqp * N;
    uint64_t* a = acc + b0 * 2 * nqp * N;
    hipLaunchKernelGGL((ntt_col_kernel<A, LOGN1, LOGN2, true, false, false>),
                       dim3((uint32_t)(nb * DN * nqp * kColBlocks)), dim3(kColNT), 0, s, e, e, twf, p->d_mods, nqp,
                       0u, nb * DN, 1u);
    hipLaunchKernelGGL((ntt_row_ks_kernel<A, LOGN1, DN, kKsRows>), dim3((uint32_t)(nb * nqp * kRowBlocks)),
                       dim3(kKsNT), 0, s, a, e, ksk, twf, twi, p->d_mods, nqp, nb);
    hipLaunchKernelGGL((ntt_col_kernel<A, LOGN1, LOGN2, false, true, false>),
                       dim3((uint32_t)(nb * 2 * nqp * kColBlocks)), dim3(kColNT), 0, s, a, a, twi, p->d_mods, nqp,
                       0u, nb * 2, 1u);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

template <class A, int LOGN1>
hipError_t launch_ks_middle_dn(const ntt_plan* p, uint64_t* acc, uint64_t* ext, const uint64_t* ksk, uint64_t batch,
                               uint32_t nqp, uint32_t dnum, hipStream_t s) {
  switch (dnum) {
    case 1: return launch_ks_middle_split<A, LOGN1, 1>(p, acc, ext, ksk, batch, nqp, s);
    case 2: return launch_ks_middle_split<A, LOGN1, 2>(p, acc, ext, ksk, batch, nqp, s);
    case 3: return launch_ks_middle_split<A, LOGN1, 3>(p, acc, ext, ksk, batch, nqp, s);
    case 4: return launch_ks_middle_split<A, LOGN1, 4>(p, acc, ext, ksk, batch, nqp, s);
    default: return hipErrorNotSupported;
  }
}

template <class A>
hipError_t launch_ks_middle_any(const ntt_plan* p, uint64_t* acc, uint64_t* ext, const uint64_t* ksk,
                                uint64_t batch, uint32_t nqp, uint32_t dnum, hipStream_t s) {
  if (p->logn == 15) return launch_ks_middle_dn<A, 7>(p, acc, ext, ksk, batch, nqp, dnum, s);
  if (p->logn == 16) return launch_ks_middle_dn<A, 8>(p, acc, ext, ksk, batch, nqp, dnum, s);
  return hipErrorNotSupported;
}

template <class A>
hipError_t launch_any(const ntt_plan* p, uint64_t* data, const uint64_t* in, uint64_t rows, uint32_t limb_begin,
                      uint32_t num_limbs, Op op, uint32_t g, hipStream_t s) {
  switch (p->logn) {
#define NNTT_CASE(L) \
  case L:            \
    return launch_lds<A, L>(p, data, in, rows, limb_begin, num_limbs, op, g, s);
    NNTT_CASE(1)
    NNTT_CASE(2)
    NNTT_CASE(3)
    NNTT_CASE(4)
    NNTT_CASE(5)
    NNTT_CASE(6)
    NNTT_CASE(7)
    NNTT_CASE(8)
    NNTT_CASE(9)
    NNTT_CASE(10)
    NNTT_CASE(11)
    NNTT_CASE(12)
    NNTT_CASE(13)
#undef NNTT_CASE
    case 14:
      // 64-bit residues take the two-pass split (128 x 128): with one 136 KiB whole-row
      // workgroup per CU nothing overlaps a row's loads and stores.  Measured on MI355X,
      // 2048 limbs of 60 bits: forward 279-286 -> 230-240 us, inverse 292-296 -> 245 us.
      // 30-bit rows (68 KiB, two workgroups per CU) keep the whole-row kernel.
      if constexpr (sizeof(typename A::T) == 8)
        return launch_split<A, 7, 7>(p, data, in, rows, limb_begin, num_limbs, op, g, s);
      return launch_lds<A, 14>(p, data, in, rows, limb_begin, num_limbs, op, g, s);
    case 15:
      return launch_split<A, 7, 8>(p, data, in, rows, limb_begin, num_limbs, op, g, s);
    case 16:
      return launch_split<A, 8, 8>(p, data, in, rows, limb_begin, num_limbs, op, g, s);
    default:
      return hipErrorInvalidValue;
  }
}

template <class A, int LOGN>
hipError_t launch_chain(const ntt_plan* p, uint64_t* out, const uint64_t* a, const uint64_t* b, uint64_t batch,
                        uint32_t limb_begin, uint32_t num_limbs, hipStream_t s) {
  constexpr int NT = ChainCfg<LOGN>::NT;
  const void* twf = tables_for<A>(p, Op::kForward);
  const void* twi = tables_for<A>(p, Op::kInverse);
  const uint64_t per = items_per_launch((uint64_t)num_limbs * NT);  // whole ciphertexts per launch
  if (per == 0) return hipErrorNotSupported;
  const uint64_t plane = (uint64_t)num_limbs << LOGN;
  for (uint64_t c0 = 0; c0 < batch; c0 += per) {
    const uint64_t nc = std::min(per, batch - c0);
    hipLaunchKernelGGL((ct_tensor_coeff_kernel<A, LOGN>), dim3((uint32_t)(nc * num_limbs)), dim3(NT), 0, s,
                       out + c0 * 3 * plane, a + c0 * 2 * plane, b + c0 * 2 * plane, twf, twi, p->d_mods, num_limbs,
                       limb_begin, nc);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <class A>
hipError_t launch_chain_any(const ntt_plan* p, uint64_t* out, const uint64_t* a, const uint64_t* b, uint64_t batch,
                            uint32_t limb_begin, uint32_t num_limbs, hipStream_t s) {
  switch (p->logn) {
#define NNTT_CHAIN(L) \
  case L:             \
    return launch_chain<A, L>(p, out, a, b, batch, limb_begin, num_limbs, s);
    NNTT_CHAIN(1)
    NNTT_CHAIN(2)
    NNTT_CHAIN(3)
    NNTT_CHAIN(4)
    NNTT_CHAIN(5)
    NNTT_CHAIN(6)
    NNTT_CHAIN(7)
    NNTT_CHAIN(8)
    NNTT_CHAIN(9)
    NNTT_CHAIN(10)
    NNTT_CHAIN(11)
    NNTT_CHAIN(12)
#undef NNTT_CHAIN
    default:
      return hipErrorNotSupported;
  }
}

// Every transform kernel runs at most n / 2 threads per limb, so a launch of whole
// polynomials stays within the launch cap; larger batches go in several launches.
hipError_t dispatch(const ntt_plan* p, uint64_t* data, const uint64_t* in, uint64_t batch, uint32_t limb_begin,
                    uint32_t num_limbs, Op op, uint32_t g, hipStream_t s) {
  if (batch * num_limbs == 0) return hipSuccess;
  const uint64_t per = items_per_launch((uint64_t)num_limbs * std::max<uint32_t>(1, p->n / 2));
  if (per == 0) return hipErrorNotSupported;
  const bool narrow = range_is_narrow(p, limb_begin, num_limbs), b60 = range_below60(p, limb_begin, num_limbs);
  for (uint64_t b0 = 0; b0 < batch; b0 += per) {
    const uint64_t rows = std::min(per, batch - b0) * num_limbs, off = b0 * num_limbs * p->n;
    hipError_t e;
    if (narrow) e = launch_any<Narrow>(p, data + off, in + off, rows, limb_begin, num_limbs, op, g, s);
    else if (b60) e = launch_any<Wide60>(p, data + off, in + off, rows, limb_begin, num_limbs, op, g, s);
    else e = launch_any<Wide>(p, data + off, in + off, rows, limb_begin, num_limbs, op, g, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

bool range_is_narrow(const ntt_plan* p, uint32_t limb_begin, uint32_t num_limbs) {
  for (uint32_t l = limb_begin; l < limb_begin + num_limbs; ++l)
    if (!p->narrow[l]) return false;
  return true;
}

bool range_below60(const ntt_plan* p, uint32_t limb_begin, uint32_t num_limbs) {
  for (uint32_t l = limb_begin; l < limb_begin + num_limbs; ++l)
    if (!p->below60[l]) return false;
  return true;
}

hipError_t launch_ntt(const ntt_plan* p, uint64_t* data, uint64_t batch, uint32_t limb_begin, uint32_t num_limbs,
                      bool inverse, hipStream_t s) {
  return dispatch(p, data, data, batch, limb_begin, num_limbs, inverse ? Op::kInverse : Op::kForward, 1u, s);
}

bool intt_mac_supported(const ntt_plan* p) { return p->logn >= 15; }

hipError_t launch_intt_mac(const ntt_plan* p, uint64_t* acc, const uint64_t* ext, const uint64_t* ksk, uint64_t batch,
                           uint32_t nqp, uint32_t dnum, uint32_t chunk, hipStream_t s) {
  if (!intt_mac_supported(p)) return hipErrorNotSupported;
  if (batch == 0) return hipSuccess;
  const MacSrc ms{ext, ksk, dnum, chunk, nullptr, nullptr, 0};
  if (range_is_narrow(p, 0, nqp)) return launch_mac_any<Narrow>(p, acc, ms, batch, nqp, s);
  if (range_below60(p, 0, nqp)) return launch_mac_any<Wide60>(p, acc, ms, batch, nqp, s);
  return launch_mac_any<Wide>(p, acc, ms, batch, nqp, s);
}

bool chain_supported(const ntt_plan* p) { return p->logn <= kChainMaxLogN; }

hipError_t launch_ct_tensor_coeff(const ntt_plan* p, uint64_t* out, const uint64_t* a, const uint64_t* b,
                                  uint64_t batch, uint32_t limb_begin, uint32_t num_limbs, hipStream_t s) {
  if (!chain_supported(p)) return hipErrorNotSupported;
  if (batch * num_limbs == 0) return hipSuccess;
  if (range_is_narrow(p, limb_begin, num_limbs))
    return launch_chain_any<Narrow>(p, out, a, b, batch, limb_begin, num_limbs, s);
  if (range_below60(p, limb_begin, num_limbs))
    return launch_chain_any<Wide60>(p, out, a, b, batch, limb_begin, num_limbs, s);
  return launch_chain_any<Wide>(p, out, a, b, batch, limb_begin, num_limbs, s);
}

bool ks_middle_supported(const ntt_plan* p, uint32_t dnum, uint32_t chunk) {
  return p->logn >= 15 && dnum >= 1 && dnum <= 4 && chunk >= dnum;
}

hipError_t launch_ks_middle(const ntt_plan* p, uint64_t* acc, uint64_t* ext, const uint64_t* ksk, uint64_t batch,
                            uint32_t nqp, uint32_t dnum, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  if (range_is_narrow(p, 0, nqp)) return launch_ks_middle_any<Narrow>(p, acc, ext, ksk, batch, nqp, dnum, s);
  if (range_below60(p, 0, nqp)) return launch_ks_middle_any<Wide60>(p, acc, ext, ksk, batch, nqp, dnum, s);
  return launch_ks_middle_any<Wide>(p, acc, ext, ksk, batch, nqp, dnum, s);
}

hipError_t launch_intt_mac_hoisted(const ntt_plan* p, uint64_t* acc, const uint64_t* ext, const uint64_t* ksk,
                                   uint64_t batch, uint32_t num_rot, uint32_t nqp, uint32_t dnum, uint32_t chunk,
                                   const HoistArgs& ha, const uint64_t* c0hat, const uint64_t* pr64, uint32_t nq,
                                   hipStream_t s) {
  if (!intt_mac_supported(p)) return hipErrorNotSupported;
  if (batch == 0) return hipSuccess;
  // the folded term is one more product per reduction, in the compile-time digit counts
  if (c0hat && (dnum >= chunk || dnum > 4)) return hipErrorInvalidValue;
  const MacSrc ms{ext, ksk, dnum, chunk, c0hat, pr64, nq};
  if (range_is_narrow(p, 0, nqp)) return launch_mac_hoisted_any<Narrow>(p, acc, ms, batch, num_rot, nqp, ha, s);
  if (range_below60(p, 0, nqp)) return launch_mac_hoisted_any<Wide60>(p, acc, ms, batch, num_rot, nqp, ha, s);
  return launch_mac_hoisted_any<Wide>(p, acc, ms, batch, num_rot, nqp, ha, s);
}

hipError_t launch_ntt_galois(const ntt_plan* p, uint64_t* out, const uint64_t* in, uint64_t g, uint64_t batch,
                             uint32_t limb_begin, uint32_t num_limbs, hipStream_t s) {
  return dispatch(p, out, in, batch, limb_begin, num_limbs, Op::kForwardGalois, (uint32_t)(g % (2ull * p->n)), s);
}

}  // namespace nntt
