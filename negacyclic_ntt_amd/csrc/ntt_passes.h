// Building blocks of the LDS-staged transform kernels for gfx950, shared by the
// transform kernels (ntt.hip) and the key-switch kernels that fuse work into a
// transform pass (keyswitch.hip).
//
// Stage numbering.  In a transform of size M = 2^m, stage sigma (0 <= sigma < m)
// has 2^sigma butterfly groups at distance M / 2^(sigma+1); the butterfly at
// position j uses table[prefix * 2^sigma + j / (2 * distance)].  Inside a workgroup,
// each thread holds one radix-2^r "set" (up to 16 residues) in registers and runs r
// stages on it; sets are exchanged through LDS between passes.
#pragma once
#include "internal.h"

namespace nntt {
namespace {


// Register radix (log2) of one pass: radix-16 sets (16 residues per thread).  On
// MI355X radix 2^2..2^5 were measured; radix 32 no longer fits the register file.
constexpr int kMaxRadixLog = 4;

// Split m stages into passes of at most kMaxRadixLog, as even as possible.
struct Sched {
  int np;
  int r[8];
  int s[8];
};
constexpr Sched make_sched(int logm) {
  Sched S{};
  S.np = logm <= kMaxRadixLog ? 1 : (logm + kMaxRadixLog - 1) / kMaxRadixLog;
  int base = logm / S.np, extra = logm % S.np, s = 0;
  for (int i = 0; i < S.np; ++i) {
    S.r[i] = base + (i < extra ? 1 : 0);
    S.s[i] = s;
    s += S.r[i];
  }
  return S;
}

// LDS rows are padded by one slot per 2^kPadShift residues (and one more per row), so
// that the strided set accesses of a pass spread over the banks.
template <class A>
constexpr int sub_stride(int m) {
  return (1 << m) + ((1 << m) >> A::kPadShift) + 1;
}

template <class A>
__device__ __forceinline__ int lpos(int pos) {
  return pos + (pos >> A::kPadShift);
}

// Work placement.  The logical block lb = xcd_local_block(b) (internal.h) gives each
// XCD one contiguous range of logical blocks, and logical blocks are ordered
// limb-major (every batch item and tile of plan limb 0, then limb 1, ...), so an XCD
// works through a contiguous group of primes and keeps their twiddle tables resident
// in its own 4 MB L2.
struct Place {
  uint64_t row;   // tensor row (batch item * num_limbs + limb)
  uint32_t limb;  // plan limb
  uint32_t tile;  // tile within the row
};
__device__ __forceinline__ Place place_block(uint32_t tiles_per_row, uint64_t batch, uint32_t num_limbs,
                                             uint32_t limb_begin) {
  const uint32_t lb = xcd_local_block(blockIdx.x, gridDim.x);
  const uint64_t t = lb / tiles_per_row;
  const uint32_t limb = (uint32_t)(t / batch);
  Place pl;
  pl.tile = lb % tiles_per_row;
  pl.row = (t % batch) * num_limbs + limb;
  pl.limb = limb_begin + limb;
  return pl;
}

// Per-sub-transform parameters seen by the pass executor.
template <class A>
struct SubParams {
  const typename A::Tw* tw;  // this prime's table (n entries)
  typename A::T q;
  uint32_t prefix;
  typename A::Tw ninv, w1n;  // last inverse stage with the scaling folded in (FOLD only)
};

// One pass: radix 2^R sets over stages [S0, S0 + R) of every sub-transform held
// in LDS.  NSUB sub-transforms of size 2^LOGM, NT threads.
// PRE: 1 requests every twiddle of a set before its LDS reads, 0 loads them as the
// butterflies need them, -1 takes the direction's default (forward 0, inverse 1).
// FOLD (inverse, S0 = 0): stage 0 is the transform's last one, prefix 1, and scales by
// n^-1 as it goes (gs_butterfly_scaled with sp.ninv and sp.w1n).
// CANON: the pass starts the transform on canonical inputs, so its first stage skips
// the butterflies' input reduction.
// PERM: the table is in the row-pass layout (internal.h): stage v, entry j of set g is
// at (prefix 2^S0) 2^v + j 2^S0 + g instead of (prefix 2^S0 + g) 2^v + j.
template <class A, bool FWD, int LOGM, int R, int S0, int NSUB, int NT, int PRE, class GetSub, bool FOLD = false,
          bool CANON = false, bool PERM = false>
__device__ __forceinline__ void run_pass(typename A::T* lds, int tid, const GetSub& get_sub) {
  using T = typename A::T;
  static_assert(!FOLD || (!FWD && S0 == 0), "the folded scaling belongs to the inverse's stage 0");
  constexpr int M = 1 << LOGM;
  constexpr int SETS_PER_SUB = M >> R;
  constexpr int TP = M >> (S0 + R);  // smallest distance in this pass
  constexpr int SPAN = M >> S0;      // extent of one group at stage S0
  constexpr int SETS = NSUB * SETS_PER_SUB;
  constexpr int STRIDE = sub_stride<A>(LOGM);
  constexpr int ITERS = (SETS + NT - 1) / NT;
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int set = tid + it * NT;
    if (SETS % NT != 0 && set >= SETS) break;  // a ragged last round: the rest wait at the barrier
    const int sub = set / SETS_PER_SUB, u = set % SETS_PER_SUB;
    const int g = u / TP, r = u % TP;
    const int pos0 = g * SPAN + r;
    T* base = lds + sub * STRIDE;
    const SubParams<A> sp = get_sub(sub);
    const T q = sp.q, two_q = q + q;
    const uint32_t pg = (sp.prefix << S0) + (uint32_t)g;
    // Table index of stage v, entry j of this set.
    auto twi = [&](int v, uint32_t j) -> uint32_t {
      return PERM ? ((sp.prefix << S0) << v) + (j << S0) + (uint32_t)g : (pg << v) + j;
    };
    T x[1 << R];
    if (FWD && PRE == 1) {
      // Forward with every twiddle of the set requested before the LDS reads.
      typename A::Tw wv[(1 << R) - 1];
#pragma unroll
      for (int v = 0; v < R; ++v)
#pragma unroll
        for (int j = 0; j < (1 << v); ++j) wv[(1 << v) - 1 + j] = sp.tw[twi(v, (uint32_t)j)];
#pragma unroll
      for (int i = 0; i < (1 << R); ++i) x[i] = base[lpos<A>(pos0 + i * TP)];
#pragma unroll
      for (int v = 0; v < R; ++v) {
        const int half = 1 << (R - 1 - v);
#pragma unroll
        for (int i = 0; i < (1 << R); ++i) {
          if (i & half) continue;
          if (CANON && v == 0)
            ct_butterfly<A, true>(x[i], x[i + half], wv[(1 << v) - 1 + (i >> (R - v))], q, two_q);
          else
            ct_butterfly<A>(x[i], x[i + half], wv[(1 << v) - 1 + (i >> (R - v))], q, two_q);
        }
      }
    } else if (FWD) {
#pragma unroll
      for (int i = 0; i < (1 << R); ++i) x[i] = base[lpos<A>(pos0 + i * TP)];
#pragma unroll
      for (int v = 0; v < R; ++v) {
        const int half = 1 << (R - 1 - v);
#pragma unroll
        for (int i = 0; i < (1 << R); ++i) {
          if (i & half) continue;
          const typename A::Tw w = sp.tw[twi(v, (uint32_t)(i >> (R - v)))];
          if (CANON && v == 0)
            ct_butterfly<A, true>(x[i], x[i + half], w, q, two_q);
          else
            ct_butterfly<A>(x[i], x[i + half], w, q, two_q);
        }
      }
    } else if (PRE == 0) {
#pragma unroll
      for (int i = 0; i < (1 << R); ++i) x[i] = base[lpos<A>(pos0 + i * TP)];
#pragma unroll
      for (int v = R - 1; v >= 0; --v) {
        const int half = 1 << (R - 1 - v);
#pragma unroll
        for (int i = 0; i < (1 << R); ++i) {
          if (i & half) continue;
          if (FOLD && v == 0)
            gs_butterfly_scaled<A>(x[i], x[i + half], sp.ninv, sp.w1n, q, two_q);
          else if (CANON && v == R - 1)
            gs_butterfly<A, true>(x[i], x[i + half], sp.tw[twi(v, (uint32_t)(i >> (R - v)))], q, two_q);
          else
            gs_butterfly<A>(x[i], x[i + half], sp.tw[twi(v, (uint32_t)(i >> (R - v)))], q, two_q);
        }
      }
    } else {
      // The inverse network needs its largest group of twiddles first: request all
      // 2^R - 1 of the set before the LDS reads so that their latency overlaps.
      // wv[(1 << v) - 1 + j] = stage v, group j.  (Measured: -4% on the inverse,
      // while the same preload slows the forward network, which starts with one.)
      typename A::Tw wv[(1 << R) - 1];
#pragma unroll
      for (int v = 0; v < R; ++v)
#pragma unroll
        for (int j = 0; j < (1 << v); ++j) wv[(1 << v) - 1 + j] = sp.tw[twi(v, (uint32_t)j)];
#pragma unroll
      for (int i = 0; i < (1 << R); ++i) x[i] = base[lpos<A>(pos0 + i * TP)];
#pragma unroll
      for (int v = R - 1; v >= 0; --v) {
        const int half = 1 << (R - 1 - v);
#pragma unroll
        for (int i = 0; i < (1 << R); ++i) {
          if (i & half) continue;
          if (FOLD && v == 0)
            gs_butterfly_scaled<A>(x[i], x[i + half], sp.ninv, sp.w1n, q, two_q);
          else if (CANON && v == R - 1)
            gs_butterfly<A, true>(x[i], x[i + half], wv[(1 << v) - 1 + (i >> (R - v))], q, two_q);
          else
            gs_butterfly<A>(x[i], x[i + half], wv[(1 << v) - 1 + (i >> (R - v))], q, two_q);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < (1 << R); ++i) base[lpos<A>(pos0 + i * TP)] = x[i];
  }
}

// All passes of a sub-transform of size 2^LOGM, forward (sigma up) or inverse
// (sigma down).  Ends with a barrier.
// FOLD (inverse only): the last pass scales by n^-1 (see run_pass).  CANON: these
// passes start the transform on canonical inputs (see run_pass).
// ROWT: the row transform of the two-pass split reading the row-pass table layout
// (its last pass, row stages kPermRowS0.., uses PERM indexing).
template <class A, bool FWD, int LOGM, int NSUB, int NT, int P, class GetSub, int PRE = -1, bool FOLD = false,
          bool CANON = false, bool ROWT = false>
__device__ __forceinline__ void run_passes(typename A::T* lds, int tid, const GetSub& get_sub) {
  constexpr Sched S = make_sched(LOGM);
  static_assert(!ROWT || (LOGM == (int)kPermRowLog && S.np == 2 && S.s[1] == (int)kPermRowS0),
                "the row-pass layout assumes rows of 2^8 in two radix-16 passes");
  if constexpr (P < S.np) {
    constexpr int idx = FWD ? P : S.np - 1 - P;
    run_pass<A, FWD, LOGM, S.r[idx], S.s[idx], NSUB, NT, PRE, GetSub, FOLD && P == S.np - 1, CANON && P == 0,
             ROWT && idx == S.np - 1>(lds, tid, get_sub);
    __syncthreads();
    run_passes<A, FWD, LOGM, NSUB, NT, P + 1, GetSub, PRE, FOLD, CANON, ROWT>(lds, tid, get_sub);
  }
}

template <class A>
__device__ __forceinline__ const typename A::Tw* table_of(const void* tw_all, uint32_t limb, uint32_t n) {
  return reinterpret_cast<const typename A::Tw*>(tw_all) + (size_t)limb * n;
}

template <class A>
__device__ __forceinline__ typename A::T modulus(const ModInfo& m) {
  return (typename A::T)m.q;
}

// Final store conversion: forward [0, 4q) -> [0, q); inverse: * n^-1 then [0, q).
// SCALED (inverse): the last stage already multiplied by n^-1; x in [0, 2q).
template <class A, bool FWD, bool SCALED = false>
__device__ __forceinline__ uint64_t finish(typename A::T x, const ModInfo& m) {
  using T = typename A::T;
  const T q = (T)m.q;
  if constexpr (SCALED) return A::widen(reduce_once<A>(x, q));
  if (FWD) {
    x = reduce_once<A>(x, q + q);
    return A::widen(reduce_once<A>(x, q));
  }
  typename A::Tw s;
  if constexpr (A::kShoupBits == 64) {
    s.w = m.n_inv;
    s.wp = m.n_inv_shoup;
  } else if constexpr (A::kShoupBits == 62) {
    s.w = m.n_inv;
    s.wp = m.n_inv_shoup60;
  } else {
    s.w = m.n_inv32;
    s.wp = m.n_inv_shoup32;
  }
  return A::widen(reduce_once<A>(A::mul(x, s, q), q));
}

// n^-1 and psi^-brv(1) n^-1 as Shoup pairs of the residue width.
template <class A>
__device__ __forceinline__ void scaled_last_stage(const ModInfo& m, typename A::Tw& ninv, typename A::Tw& w1n) {
  if constexpr (A::kShoupBits == 64) {
    ninv.w = m.n_inv, ninv.wp = m.n_inv_shoup;
    w1n.w = m.w1n, w1n.wp = m.w1n_shoup;
  } else if constexpr (A::kShoupBits == 62) {
    ninv.w = m.n_inv, ninv.wp = m.n_inv_shoup60;
    w1n.w = m.w1n, w1n.wp = m.w1n_shoup60;
  } else {
    ninv.w = m.n_inv32, ninv.wp = m.n_inv_shoup32;
    w1n.w = m.w1n32, w1n.wp = m.w1n_shoup32;
  }
}


// A 16-byte load, non-temporal when NT (data read once per launch).
template <bool NT>
__device__ __forceinline__ ulonglong2 load_tile(const uint64_t* p) {
  if constexpr (NT) {
    typedef unsigned long long u64x2_t __attribute__((ext_vector_type(2)));
    const u64x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u64x2_t*>(p));
    return ulonglong2{v.x, v.y};
  } else {
    return *reinterpret_cast<const ulonglong2*>(p);
  }
}

// ---------------------------------------------------------------------------
// Two-pass split for n = N1 * N2 (N2 contiguous).  Column kernel: a workgroup
// owns COLS adjacent columns (COLS * 8 B = one 128 B line per row) of one limb.
// Row kernel: a workgroup owns ROWS consecutive rows of one limb.
constexpr int kCols = 16;
constexpr int kRows = 16;

template <int LOGN1>
struct ColCfg {
  static constexpr Sched S = make_sched(LOGN1);
  static constexpr int NT = (kCols << LOGN1) >> S.r[0];
};
template <int LOGN2>
struct RowCfg {
  static constexpr Sched S = make_sched(LOGN2);
  static constexpr int NT = (kRows << LOGN2) >> S.r[0];
};

}  // namespace
}  // namespace nntt
