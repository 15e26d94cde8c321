// Hybrid rotation key-switch on gfx950.
//
// For a ciphertext (c0, c1) over Q = q_0..q_{L-1}, special primes P = p_0..p_{K-1}
// and dnum digits of alpha = L / dnum consecutive primes:
//   1. c' = sigma_g(c): the automorphism X -> X^g (coefficient domain), gathered
//      on load inside steps 2 and 6 (no separate pass over memory);
//   2. ModUp: digit j of c1' is lifted to the unique integer D_j in [0, Q_j)
//      (Garner / mixed radix -- the "mixed-radix decomposition and basis
//      extension" of FHElium "Eager, Compile, and native execution", section
//      "CUDA execution"; the "Garner extension" of the kestrel-llm overview,
//      section 4.2) and reduced onto every prime of Q u P;
//   3. forward NTT of every extended digit;
//   4. key inner product acc_c = sum_j NTT(D_j) * ksk[j][c] (FHElium's key-switch
//      multiply-accumulate);
//   5. the inverse NTT of both accumulators.  For n >= 2^15 with up to 4 digits, one
//      kernel per row tile runs the forward row pass of every digit, the key product
//      and the inverse row pass (ntt.hip, ntt_row_ks_kernel), between the two column
//      passes; with more digits the key product rides on the inverse's row pass;
//      smaller rings use mac_kernel between the transforms;
//   6. ModDown (exact floor, FHElium's "QP-to-Q ModDown"):
//      out_c = floor(X_c / P) mod q_l = (acc_c[l] - (X_c mod P)) * P^-1 mod q_l,
//      X_c mod P from the P residues by Garner; out_0 += sigma_g(c0).
// Garner: with residues x_i modulo m_i, the mixed-radix digits are
//   v_i = (x_i - sum_{k<i} v_k prod_{j<k} m_j) * (prod_{j<i} m_j)^-1  mod m_i,
// and D = sum_i v_i prod_{j<i} m_j lies in [0, prod m_i); D mod p is then
// sum_i v_i (prod_{j<i} m_j mod p).  Below 2^60 the sums of products by plan
// constants are 30-bit-half dot products with one Montgomery reduction (dot30);
// otherwise each product is a Shoup product with partial sums kept in [0, 2p).
// The extended digits are stored times 2^64 (Montgomery form) so that the key
// product needs one Montgomery reduction per output.
#include <string.h>

#include <algorithm>
#include <new>

#include "ntt_passes.h"
#include "rns.h"

namespace nntt {
namespace {

constexpr int kKsThreads = 256;
// Launch shapes measured on MI355X (n = 2^16, 24 + 8 primes below 2^60, dnum 3):
// ModUp over all target primes in one group (the exact-width Garner chain needs no
// extra waves: 28.8 us, two groups 29.6, four 40); ModDown in two groups of output
// primes (one: 32, three: 30 us) whose loads are issued four limbs at a time (24.6 us;
// eight: 25.7, twelve: 29.8).  Primes at or above 2^60 keep two ModUp groups.
constexpr uint32_t kModUpGroups = 1;
constexpr uint32_t kModUpGroupsWide = 2;
constexpr uint32_t kModDownGroups = 2;
constexpr int kModDownChunk = 4;
// The residue-number-system helpers (Garner, evaluations, the automorphism gather,
// the plan constants) are in rns.h.

// ---- ModUp with the automorphism fused on load ---------------------------------
// grid.x: coefficient tiles; grid.y: batch * dnum; grid.z: groups of target primes.
// Each thread lifts one coefficient of one digit (Garner) and reduces it onto its
// group's share of the nq + np - alpha other primes: the groups multiply the
// number of resident waves (the Garner digits are recomputed per group).
// ext: [batch][dnum][nq+np][n], in Montgomery form: D_j 2^64 mod q_t (the evaluation
// constants carry the factor 2^64; the digit's own residues are scaled by one Shoup
// product), so that the key product needs a single Montgomery reduction per output.
// src: the polynomial that is decomposed, [batch][nq][n] with batch stride src_stride
// (c1 of a ciphertext, or d2 of a tensor product).
// EX = K: the launch has exactly K primes per digit, so the loops over them have
// compile-time bounds (one straight-line block the scheduler can interleave).
template <bool B60, int K, bool EX>
__global__ __launch_bounds__(kKsThreads) void modup_kernel(uint64_t* __restrict__ ext,
                                                           const uint64_t* __restrict__ src, uint64_t src_stride,
                                                           KsDev kc, uint32_t logn, uint32_t h, uint32_t nq,
                                                           uint32_t np_, uint32_t alpha_arg, uint32_t dnum) {
  const uint32_t alpha = EX ? (uint32_t)K : alpha_arg;
  const uint32_t n = 1u << logn;
  const uint32_t e = blockIdx.x * kKsThreads + threadIdx.x;
  if (e >= n) return;
  const uint32_t bj = blockIdx.y, b = bj / dnum, j = bj % dnum;
  const uint32_t nqp = nq + np_;
  const uint64_t* c1 = src + (uint64_t)b * src_stride;
  const Gather gi = gather_index(e, h, logn);
  const uint32_t first = j * alpha;
  uint64_t x[K], v[K];
#pragma unroll
  for (int i = 0; i < K; ++i) {
    if (i >= (int)alpha) break;
    const uint64_t q = kc.moduli[first + i];
    const uint64_t a = c1[(uint64_t)(first + i) * n + gi.src];
    x[i] = gi.neg ? neg_mod(a, q) : a;
  }
  uint64_t* out = ext + (uint64_t)bj * nqp * n + e;
  if (blockIdx.z == 0) {
#pragma unroll
    for (int i = 0; i < K; ++i) {
      if (i >= (int)alpha) break;
      const uint64_t q = kc.moduli[first + i];  // the digit's own primes keep their residues
      out[(uint64_t)(first + i) * n] = csub(shoup<B60>(x[i], kc.r_scale[first + i], q), q);
    }
  }
  constexpr int S = kMaxDigitPrimes;
  uint32_t vl[K], vh[K];
  if constexpr (B60)
    garner30<K, S>(x, v, vl, vh, alpha, kc.moduli + first, kc.ninv + first, kc.digit_garner + (size_t)j * S * S,
                   kc.digit_garner30 + (size_t)j * S * S);
  else
    garner<B60, K, S>(x, v, alpha, kc.moduli + first, kc.digit_garner + (size_t)j * S * S);
  const Tw* ev = kc.digit_eval + (size_t)j * nqp * S;
  // targets m = 0 .. nqp - alpha - 1 skip the digit's own primes: t = m or m + alpha
  const uint32_t others = nqp - alpha, per = (others + gridDim.z - 1) / gridDim.z;
  const uint32_t m0 = blockIdx.z * per, m1 = min(others, m0 + per);
  if constexpr (B60) {
    const C30* ev30 = kc.digit_eval30 + (size_t)j * nqp * S;
#pragma unroll 2
    for (uint32_t m = m0; m < m1; ++m) {
      const uint32_t t = m < first ? m : m + alpha;
      out[(uint64_t)t * n] = dot30<K>(vl, vh, alpha, ev30 + (size_t)t * S, kc.moduli[t], kc.ninv[t]);
    }
  } else {
#pragma unroll 4
    for (uint32_t m = m0; m < m1; ++m) {
      const uint32_t t = m < first ? m : m + alpha;
      out[(uint64_t)t * n] = mixed_radix_eval<B60, K>(v, alpha, ev + (size_t)t * S, kc.moduli[t]);
    }
  }
}

// ---- key inner product -----------------------------------------------------------
// (Rings below 2^15; larger rings fuse this product into the inverse NTT, ntt.hip.)
// acc[b][c][t][e] = sum_j ext[b][j][t][e] * ksk[j][c][t][e]  (mod q_t), two coefficients
// per thread.  The digits carry a factor 2^64, so the exact 128-bit sum of up to
// `chunk` products (chunk q_t <= 2^64 keeps it below q_t 2^64) is Montgomery-reduced
// once to the plain residue.
struct MacSum {
  Acc128 t{0, 0};
  uint64_t r = 0;  // reduced chunks, canonical
  __device__ __forceinline__ void fold(uint64_t q, uint64_t ninv) {
    r = add_mod(r, csub(redc(t, q, ninv), q), q);
    t = Acc128{0, 0};
  }
};

__global__ __launch_bounds__(kKsThreads) void mac_kernel(uint64_t* __restrict__ acc, const uint64_t* __restrict__ ext,
                                                         const uint64_t* __restrict__ ksk,
                                                         const ModInfo* __restrict__ mods, uint32_t logn,
                                                         uint32_t nqp, uint32_t dnum, uint32_t chunk,
                                                         uint64_t pairs_per_batch) {
  const uint64_t p = (uint64_t)blockIdx.x * kKsThreads + threadIdx.x;
  const uint32_t b = blockIdx.y;
  if (p >= pairs_per_batch) return;
  const uint64_t off = 2 * p;  // index in [nqp][n]
  const uint32_t t = (uint32_t)(off >> logn);
  const uint64_t q = mods[t].q, ninv = mods[t].mont_ninv;
  const uint64_t plane = (uint64_t)nqp << logn;
  const uint64_t* xe = ext + (uint64_t)b * dnum * plane + off;
  MacSum s0x, s0y, s1x, s1y;
  uint32_t c = 0;
  for (uint32_t j = 0; j < dnum; ++j) {
    const ulonglong2 d = *reinterpret_cast<const ulonglong2*>(xe + (uint64_t)j * plane);
    const ulonglong2 k0 = *reinterpret_cast<const ulonglong2*>(ksk + ((uint64_t)j * 2) * plane + off);
    const ulonglong2 k1 = *reinterpret_cast<const ulonglong2*>(ksk + ((uint64_t)j * 2 + 1) * plane + off);
    mac128(s0x.t, d.x, k0.x);
    mac128(s0y.t, d.y, k0.y);
    mac128(s1x.t, d.x, k1.x);
    mac128(s1y.t, d.y, k1.y);
    if (++c == chunk || j + 1 == dnum) {
      s0x.fold(q, ninv);
      s0y.fold(q, ninv);
      s1x.fold(q, ninv);
      s1y.fold(q, ninv);
      c = 0;
    }
  }
  uint64_t* o = acc + (uint64_t)b * 2 * plane + off;
  *reinterpret_cast<ulonglong2*>(o) = ulonglong2{s0x.r, s0y.r};
  *reinterpret_cast<ulonglong2*>(o + plane) = ulonglong2{s1x.r, s1y.r};
}

// ---- key inner product for hoisted rotations -------------------------------------------
// (Rings below 2^15; larger rings fuse this product into the inverse NTT, ntt.hip.)
// One block owns an aligned segment S of one limb of the NTT-domain digits and stages
// it in LDS for all dnum digits; for rotation r it then produces the output segment
// slot_r^-1(S) = slot_{h_r}(S), reading the key and writing the accumulators with
// coalesced 16-byte accesses and gathering the digits from LDS.  The digits are read
// from HBM once for all R rotations.
// grid.x: nseg * nqp; grid.y: batch.  acc: [R][batch][2][nqp][n].
__global__ __launch_bounds__(kKsThreads) void mac_hoisted_kernel(uint64_t* __restrict__ acc,
                                                                 const uint64_t* __restrict__ ext,
                                                                 const uint64_t* __restrict__ ksk,
                                                                 const ModInfo* __restrict__ mods, uint32_t logn,
                                                                 uint32_t seglog, uint32_t nqp, uint32_t dnum,
                                                                 uint32_t chunk, uint32_t R, uint32_t batch,
                                                                 HoistArgs ha) {
  extern __shared__ uint64_t seg_lds[];  // [dnum][seg]
  const uint32_t seg = 1u << seglog, nseg = 1u << (logn - seglog);
  const uint32_t t = blockIdx.x >> (logn - seglog), s0 = (blockIdx.x & (nseg - 1)) << seglog;
  const uint32_t b = blockIdx.y;
  const uint64_t plane = (uint64_t)nqp << logn;
  const uint64_t row = (uint64_t)t << logn;
  const uint32_t i2 = 2 * threadIdx.x;
  const bool active = i2 < seg;
  if (active) {
    const uint64_t* xe = ext + (uint64_t)b * dnum * plane + row + s0 + i2;
    for (uint32_t j = 0; j < dnum; ++j) {
      const ulonglong2 v = *reinterpret_cast<const ulonglong2*>(xe + (uint64_t)j * plane);
      seg_lds[j * seg + i2] = v.x;
      seg_lds[j * seg + i2 + 1] = v.y;
    }
  }
  __syncthreads();
  if (!active) return;
  const uint64_t q = mods[t].q, ninv = mods[t].mont_ninv;
#pragma unroll 2
  for (uint32_t r = 0; r < R; ++r) {
    const uint32_t g = ha.g[r];
    const uint32_t k0 = (ntt_slot(s0, ha.h[r], logn) & ~(seg - 1)) + i2;
    const uint32_t p0 = ntt_slot(k0, g, logn) - s0, p1 = ntt_slot(k0 + 1, g, logn) - s0;
    const uint64_t* kr = ksk + (uint64_t)r * dnum * 2 * plane + row + k0;
    MacSum s0x, s0y, s1x, s1y;
    uint32_t c = 0;
    for (uint32_t j = 0; j < dnum; ++j) {
      const uint64_t d0 = seg_lds[j * seg + p0], d1 = seg_lds[j * seg + p1];
      const ulonglong2 k0v = *reinterpret_cast<const ulonglong2*>(kr + (uint64_t)(2 * j) * plane);
      const ulonglong2 k1v = *reinterpret_cast<const ulonglong2*>(kr + (uint64_t)(2 * j + 1) * plane);
      mac128(s0x.t, d0, k0v.x);
      mac128(s0y.t, d1, k0v.y);
      mac128(s1x.t, d0, k1v.x);
      mac128(s1y.t, d1, k1v.y);
      if (++c == chunk || j + 1 == dnum) {
        s0x.fold(q, ninv);
        s0y.fold(q, ninv);
        s1x.fold(q, ninv);
        s1y.fold(q, ninv);
        c = 0;
      }
    }
    uint64_t* o = acc + ((uint64_t)r * batch + b) * 2 * plane + row + k0;
    *reinterpret_cast<ulonglong2*>(o) = ulonglong2{s0x.r, s0y.r};
    *reinterpret_cast<ulonglong2*>(o + plane) = ulonglong2{s1x.r, s1y.r};
  }
}

// ---- ModDown + the additive part -----------------------------------------------------
// grid.x: coefficient tiles; grid.y: batch * 2 (component); grid.z: groups of the nq
// output primes (the Garner digits over P are recomputed per group).
// acc: [batch][2][nq+np][n].  Output component c gets sigma_g(add[b][c]) added when
// bit c of add_mask is set (add: [batch][*][nq][n], batch stride add_stride): c0 for
// a rotation, (d0, d1) for a relinearisation.
// grid.z = rotations x groups: rotation r (hoisted rotations; 0 otherwise) reads
// acc + r acc_rot, writes out + r out_rot and gathers the additive input through
// sigma with h = ha.h[r].
// EX = KP: exactly KP special primes (compile-time loop bounds, as in modup_kernel).
template <bool B60, int KP, bool EX>
__global__ __launch_bounds__(kKsThreads) void moddown_kernel(uint64_t* __restrict__ out,
                                                             const uint64_t* __restrict__ acc,
                                                             const uint64_t* __restrict__ add, uint64_t add_stride,
                                                             uint32_t add_mask, KsDev kc, uint32_t logn, uint32_t nq,
                                                             uint32_t np_arg, uint32_t groups, uint64_t out_rot,
                                                             uint64_t acc_rot, HoistArgs ha) {
  const uint32_t np_ = EX ? (uint32_t)KP : np_arg;
  const uint32_t n = 1u << logn;
  const uint32_t e = blockIdx.x * kKsThreads + threadIdx.x;
  if (e >= n) return;
  const uint32_t rot = blockIdx.z / groups, grp = blockIdx.z % groups;
  const uint32_t h = ha.h[rot];
  out += rot * out_rot;
  acc += rot * acc_rot;
  const uint32_t bc = blockIdx.y, b = bc >> 1, comp = bc & 1;
  const uint32_t nqp = nq + np_;
  const uint64_t* a = acc + (uint64_t)bc * nqp * n + e;
  uint64_t y[KP], v[KP];
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    if (i >= (int)np_) break;
    y[i] = a[(uint64_t)(nq + i) * n];
  }
  const bool adds = (add_mask >> comp) & 1u;
  const uint64_t* c0 = add + (uint64_t)b * add_stride + (uint64_t)comp * nq * n;
  const Gather gi = gather_index(e, h, logn);
  uint64_t* o = out + (uint64_t)bc * nq * n + e;
  const uint32_t per = (nq + groups - 1) / groups;
  const uint32_t l0 = grp * per, l1 = min(nq, l0 + per);
  // The output limbs go in chunks whose loads (accumulator residue, gathered addend)
  // are all issued together; the first chunk's before the Garner digits are computed.
  constexpr int CH = kModDownChunk;
  uint64_t av[CH], cv[CH];
  auto prefetch = [&](uint32_t lb) {
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const uint32_t l = lb + k;
      if (l < l1) {
        av[k] = a[(uint64_t)l * n];
        cv[k] = adds ? c0[(uint64_t)l * n + gi.src] : 0;
      }
    }
  };
  prefetch(l0);
  constexpr int S = kMaxSpecial;
  uint32_t vl[KP], vh[KP];
  if constexpr (B60)
    garner30<KP, S>(y, v, vl, vh, np_, kc.moduli + nq, kc.ninv + nq, kc.p_garner, kc.p_garner30);
  else
    garner<B60, KP, S>(y, v, np_, kc.moduli + nq, kc.p_garner);
  for (uint32_t lb = l0; lb < l1; lb += CH) {
    if (lb != l0) prefetch(lb);
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const uint32_t l = lb + k;
      if (l >= l1) break;
      const uint64_t q = kc.moduli[l];
      uint64_t r;  // (X mod P) mod q_l
      if constexpr (B60) r = dot30<KP>(vl, vh, np_, kc.p_eval30 + (size_t)l * S, q, kc.ninv[l]);
      else r = mixed_radix_eval<B60, KP>(v, np_, kc.p_eval + (size_t)l * S, q);
      const uint64_t d = sub_mod(av[k], r, q);
      uint64_t res = csub(shoup<B60>(d, kc.p_inv[l], q), q);
      if (adds) res = add_mod(res, gi.neg ? neg_mod(cv[k], q) : cv[k], q);
      o[(uint64_t)l * n] = res;
    }
  }
}

// ---- ModRaise ---------------------------------------------------------------------------
// The exact Garner lift of each coefficient from the first `from` primes, reduced onto
// primes from .. to-1 (the kestrel-llm bootstrapping profile's first stage).
// grid.x: coefficient tiles; grid.y: batch; grid.z: groups of target primes.
// in: [batch][from][n]; out: [batch][to][n].
template <bool B60, int K>
__global__ __launch_bounds__(kKsThreads) void modraise_kernel(uint64_t* __restrict__ out,
                                                              const uint64_t* __restrict__ in,
                                                              const uint64_t* __restrict__ moduli,
                                                              const Tw* __restrict__ gar, const Tw* __restrict__ ev,
                                                              uint32_t logn, uint32_t from, uint32_t to) {
  const uint32_t n = 1u << logn;
  const uint32_t e = blockIdx.x * kKsThreads + threadIdx.x;
  if (e >= n) return;
  const uint64_t* x_in = in + (uint64_t)blockIdx.y * from * n + e;
  uint64_t* o = out + (uint64_t)blockIdx.y * to * n + e;
  uint64_t x[K], v[K];
#pragma unroll
  for (int i = 0; i < K; ++i) {
    if (i >= (int)from) break;
    x[i] = x_in[(uint64_t)i * n];
  }
  if (blockIdx.z == 0) {
#pragma unroll
    for (int i = 0; i < K; ++i) {
      if (i >= (int)from) break;
      o[(uint64_t)i * n] = x[i];
    }
  }
  constexpr int S = kMaxDigitPrimes;
  garner<B60, K, S>(x, v, from, moduli, gar);
  const uint32_t others = to - from, per = (others + gridDim.z - 1) / gridDim.z;
  const uint32_t m0 = blockIdx.z * per, m1 = min(others, m0 + per);
#pragma unroll 4
  for (uint32_t m = m0; m < m1; ++m) {
    const uint32_t t = from + m;
    o[(uint64_t)t * n] = mixed_radix_eval<B60, K>(v, from, ev + (size_t)t * S, moduli[t]);
  }
}

}  // namespace
}  // namespace nntt

using namespace nntt;

struct ntt_ks_plan {
  const ntt_plan* qp = nullptr;
  uint32_t nq = 0, np = 0, dnum = 0, alpha = 0;
  uint32_t mac_chunk = 1;  // products summed before a Montgomery reduction: chunk q < 2^64
  uint32_t mac_chunk_max = 1;  // the same bound without the cap at dnum (at most 64)
  bool below60 = false;    // every prime of Q u P below 2^60
  void* d_const = nullptr;
  KsDev dev{};
};

namespace {

Tw shoup_pair(uint64_t w, uint64_t q) {
  return Tw{w, (uint64_t)(((unsigned __int128)w << 64) / q)};
}

// g[i * K + k]: prod_{j<k} m_j mod m_i (k < i), and (prod_{j<i} m_j)^-1 mod m_i (k == i).
void garner_table(const uint64_t* m, uint32_t k, uint32_t K, Tw* g) {
  for (uint32_t i = 0; i < k; ++i) {
    uint64_t prod = 1 % m[i];
    for (uint32_t kk = 0; kk < i; ++kk) {
      g[i * K + kk] = shoup_pair(prod, m[i]);
      prod = host_mulmod(prod, m[kk] % m[i], m[i]);
    }
    g[i * K + i] = shoup_pair(i ? host_invmod(prod, m[i]) : 1 % m[i], m[i]);
  }
}

// c[i] = scale * prod_{j<i} m_j mod p
void eval_table(const uint64_t* m, uint32_t k, uint64_t p, Tw* c, uint64_t scale = 1) {
  uint64_t prod = scale % p;
  for (uint32_t i = 0; i < k; ++i) {
    c[i] = shoup_pair(prod, p);
    prod = host_mulmod(prod, m[i] % p, p);
  }
}

}  // namespace

extern "C" int keyswitch_plan_create(ntt_ks_plan** out, const ntt_plan* qp, uint32_t nq, uint32_t np_,
                                     uint32_t dnum) {
  if (!out) return NTT_EINVAL;
  *out = nullptr;
  if (!qp) return NTT_EINVAL;
  if (qp->device < 0) return NTT_EDEVICE;
  if (nq == 0 || np_ == 0 || dnum == 0 || nq % dnum != 0 || nq + np_ > qp->num_primes) return NTT_EINVAL;
  const uint32_t alpha = nq / dnum;
  if (alpha > (uint32_t)kMaxDigitPrimes || np_ > (uint32_t)kMaxSpecial) return NTT_EUNSUPPORTED;
  const uint32_t nqp = nq + np_, K = (uint32_t)kMaxDigitPrimes, KP = (uint32_t)kMaxSpecial;
  const uint64_t* m = qp->primes.data();

  std::vector<uint64_t> moduli(m, m + nqp);
  std::vector<Tw> dg((size_t)dnum * K * K, Tw{0, 0}), de((size_t)dnum * nqp * K, Tw{0, 0});
  std::vector<Tw> pg((size_t)KP * KP, Tw{0, 0}), pe((size_t)nq * KP, Tw{0, 0}), pinv(nq), rs(nqp);
  std::vector<uint64_t> pr64(nq);
  uint64_t qmax = 0;
  for (uint32_t t = 0; t < nqp; ++t) {
    rs[t] = shoup_pair((uint64_t)(((unsigned __int128)1 << 64) % m[t]), m[t]);  // 2^64 mod q_t
    qmax = std::max(qmax, m[t]);
  }
  for (uint32_t j = 0; j < dnum; ++j) {
    garner_table(m + j * alpha, alpha, K, dg.data() + (size_t)j * K * K);
    for (uint32_t t = 0; t < nqp; ++t)  // digits are written in Montgomery form (times 2^64)
      eval_table(m + j * alpha, alpha, m[t], de.data() + ((size_t)j * nqp + t) * K, rs[t].w);
  }
  // Below 2^60 the evaluations use 30-bit halves and one Montgomery reduction, which
  // divides by 2^64: the digit constants carry 2^128 (result times 2^64), P's 2^64.
  std::vector<C30> de30((size_t)dnum * nqp * K, C30{0, 0}), pe30((size_t)nq * KP, C30{0, 0});
  std::vector<uint64_t> ninv(nqp);
  auto split = [](uint64_t c) { return C30{(uint32_t)(c & 0x3fffffffu), (uint32_t)(c >> 30)}; };
  for (uint32_t t = 0; t < nqp; ++t) ninv[t] = qp->h_mods[t].mont_ninv;
  std::vector<C30> dg30((size_t)dnum * K * K, C30{0, 0}), pg30((size_t)KP * KP, C30{0, 0});
  if (range_below60(qp, 0, nqp)) {
    for (size_t i = 0; i < de30.size(); ++i) {
      const uint32_t t = (uint32_t)((i / K) % nqp);
      de30[i] = split(host_mulmod(de[i].w, rs[t].w, m[t]));
    }
    for (uint32_t j = 0; j < dnum; ++j)  // below-diagonal Garner constants of digit j, times 2^64
      for (uint32_t i = 1; i < alpha; ++i)
        for (uint32_t kk = 0; kk < i; ++kk) {
          const size_t idx = ((size_t)j * K + i) * K + kk;
          const uint32_t t = j * alpha + i;
          dg30[idx] = split(host_mulmod(dg[idx].w, rs[t].w, m[t]));
        }
  }
  garner_table(m + nq, np_, KP, pg.data());
  if (range_below60(qp, 0, nqp))
    for (uint32_t i = 1; i < np_; ++i)
      for (uint32_t kk = 0; kk < i; ++kk)
        pg30[(size_t)i * KP + kk] = split(host_mulmod(pg[(size_t)i * KP + kk].w, rs[nq + i].w, m[nq + i]));
  for (uint32_t l = 0; l < nq; ++l) {
    eval_table(m + nq, np_, m[l], pe.data() + (size_t)l * KP);
    if (range_below60(qp, 0, nqp))
      for (uint32_t i = 0; i < np_; ++i)
        pe30[(size_t)l * KP + i] = split(host_mulmod(pe[(size_t)l * KP + i].w, rs[l].w, m[l]));
    uint64_t P = 1;
    for (uint32_t i = 0; i < np_; ++i) P = host_mulmod(P, m[nq + i] % m[l], m[l]);
    pinv[l] = shoup_pair(host_invmod(P, m[l]), m[l]);
    pr64[l] = host_mulmod(P, rs[l].w, m[l]);  // P 2^64 mod q_l
  }

  const size_t sz_m = moduli.size() * 8, sz_dg = dg.size() * sizeof(Tw), sz_de = de.size() * sizeof(Tw);
  const size_t sz_pg = pg.size() * sizeof(Tw), sz_pe = pe.size() * sizeof(Tw), sz_pi = pinv.size() * sizeof(Tw);
  const size_t sz_rs = rs.size() * sizeof(Tw), sz_d30 = de30.size() * sizeof(C30), sz_p30 = pe30.size() * sizeof(C30);
  const size_t sz_ni = ninv.size() * 8, sz_dg30 = dg30.size() * sizeof(C30), sz_pg30 = pg30.size() * sizeof(C30);
  const size_t sz_pr = pr64.size() * 8;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  constexpr int kParts = 13;
  const void* src[kParts] = {moduli.data(), dg.data(),   de.data(),   pg.data(),   pe.data(),   pinv.data(), rs.data(),
                             de30.data(),   pe30.data(), ninv.data(), dg30.data(), pg30.data(), pr64.data()};
  const size_t sz[kParts] = {sz_m,   sz_dg,  sz_de, sz_pg,   sz_pe,   sz_pi, sz_rs,
                             sz_d30, sz_p30, sz_ni, sz_dg30, sz_pg30, sz_pr};
  size_t total = 0;
  for (int i = 0; i < kParts; ++i) total += al(sz[i]);
  std::vector<uint8_t> blob(total, 0);
  size_t off[kParts], o = 0;
  for (int i = 0; i < kParts; ++i) {
    off[i] = o;
    memcpy(blob.data() + o, src[i], sz[i]);
    o += al(sz[i]);
  }

  ntt_ks_plan* p = new (std::nothrow) ntt_ks_plan;
  if (!p) return NTT_ENOMEM;
  {
    DeviceGuard g(qp->device);
    if (!g.ok) {
      delete p;
      return NTT_EDEVICE;
    }
    if (hipMalloc(&p->d_const, total) != hipSuccess) {
      delete p;
      return NTT_ENOMEM;
    }
    if (hipMemcpy(p->d_const, blob.data(), total, hipMemcpyHostToDevice) != hipSuccess) {
      (void)hipFree(p->d_const);
      delete p;
      return NTT_EDEVICE;
    }
  }
  uint8_t* base = (uint8_t*)p->d_const;
  p->qp = qp;
  p->nq = nq;
  p->np = np_;
  p->dnum = dnum;
  p->alpha = alpha;
  p->below60 = range_below60(qp, 0, nqp);
  p->dev.moduli = (const uint64_t*)(base + off[0]);
  p->dev.digit_garner = (const Tw*)(base + off[1]);
  p->dev.digit_eval = (const Tw*)(base + off[2]);
  p->dev.p_garner = (const Tw*)(base + off[3]);
  p->dev.p_eval = (const Tw*)(base + off[4]);
  p->dev.p_inv = (const Tw*)(base + off[5]);
  p->dev.r_scale = (const Tw*)(base + off[6]);
  p->dev.digit_eval30 = (const C30*)(base + off[7]);
  p->dev.p_eval30 = (const C30*)(base + off[8]);
  p->dev.ninv = (const uint64_t*)(base + off[9]);
  p->dev.digit_garner30 = (const C30*)(base + off[10]);
  p->dev.p_garner30 = (const C30*)(base + off[11]);
  p->dev.p_r64 = (const uint64_t*)(base + off[12]);
  p->mac_chunk = (uint32_t)std::min<uint64_t>(dnum, ~0ull / qmax);
  p->mac_chunk_max = (uint32_t)std::min<uint64_t>(64, ~0ull / qmax);
  *out = p;
  return NTT_OK;
}

int nntt::ks_plan_device(const ntt_ks_plan* p) { return p->qp->device; }

static uint64_t ws_elems(const ntt_ks_plan* p, uint64_t batch) {
  return batch * (uint64_t)(p->dnum + 2) * (p->nq + p->np) * p->qp->n;
}

extern "C" int keyswitch_workspace_size(const ntt_ks_plan* p, uint64_t batch, size_t* bytes) {
  if (!p || !bytes) return NTT_EINVAL;
  if (batch > 4096) return NTT_EUNSUPPORTED;
  *bytes = (size_t)ws_elems(p, batch) * 8;
  return NTT_OK;
}

namespace {
bool ranges_overlap(const void* a, uint64_t na, const void* b, uint64_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return na && nb && x < y + nb && y < x + na;
}

// What one key-switch pipeline reads besides the key: the decomposed polynomial and
// the polynomials added to the ModDown output (both gathered through sigma_g).
struct KsIo {
  const uint64_t* src;  // first batch's decomposed polynomial
  uint64_t src_stride;  // elements between batches
  const uint64_t* add;  // first batch's component 0 of the additive input
  uint64_t add_stride;
  uint32_t add_mask;  // bit c: add component c to output c
  uint64_t in_bytes;  // whole input extent, for the overlap checks
  const uint64_t* in;
};

// Debug input checks of a key-switch call: rows of the input over Q, rows of the key over Q u P.
int ks_debug_inputs(const ntt_ks_plan* p, const uint64_t* in, uint64_t in_rows, const uint64_t* key,
                    uint64_t key_rows, hipStream_t s) {
  int rc = debug_check_inputs(p->qp, in, in_rows, 0, p->nq, s);
  if (rc == NTT_OK) rc = debug_check_inputs(p->qp, key, key_rows, 0, p->nq + p->np, s);
  return rc;
}

// Validation shared by the entry points; returns NTT_OK or the error.
int ks_check(const ntt_ks_plan* p, uint64_t* out, const KsIo& io, const uint64_t* ksk, uint64_t batch,
             void* workspace, size_t workspace_bytes) {
  const ntt_plan* qp = p->qp;
  const uint32_t n = qp->n, nq = p->nq, nqp = nq + p->np;
  if (batch > 4096) return NTT_EUNSUPPORTED;
  if (!out || !io.in || !ksk || !workspace) return NTT_EINVAL;
  if (((uintptr_t)out | (uintptr_t)io.in | (uintptr_t)ksk) & 15u) return NTT_EINVAL;
  if ((uintptr_t)workspace & 255u) return NTT_EINVAL;
  const uint64_t need = ws_elems(p, batch) * 8;
  if (workspace_bytes < need) return NTT_EINVAL;
  const uint64_t out_bytes = batch * 2ull * nq * n * 8, ksk_bytes = (uint64_t)p->dnum * 2 * nqp * n * 8;
  if (ranges_overlap(out, out_bytes, io.in, io.in_bytes) || ranges_overlap(out, out_bytes, ksk, ksk_bytes) ||
      ranges_overlap(out, out_bytes, workspace, need) || ranges_overlap(workspace, need, io.in, io.in_bytes) ||
      ranges_overlap(workspace, need, ksk, ksk_bytes))
    return NTT_EOVERLAP;
  return NTT_OK;
}

template <bool B60, int K>
void launch_modup(dim3 grid, hipStream_t s, uint64_t* ext, const KsIo& io, const ntt_ks_plan* p, uint32_t h) {
  if (p->alpha == (uint32_t)K)
    hipLaunchKernelGGL((modup_kernel<B60, K, true>), grid, dim3(kKsThreads), 0, s, ext, io.src, io.src_stride,
                       p->dev, p->qp->logn, h, p->nq, p->np, p->alpha, p->dnum);
  else
    hipLaunchKernelGGL((modup_kernel<B60, K, false>), grid, dim3(kKsThreads), 0, s, ext, io.src, io.src_stride,
                       p->dev, p->qp->logn, h, p->nq, p->np, p->alpha, p->dnum);
}

template <bool B60, int KP>
void launch_moddown(dim3 grid, hipStream_t s, uint64_t* out, const uint64_t* acc, const KsIo& io,
                    const ntt_ks_plan* p, uint32_t groups, uint64_t out_rot, uint64_t acc_rot, const HoistArgs& ha) {
  if (p->np == (uint32_t)KP)
    hipLaunchKernelGGL((moddown_kernel<B60, KP, true>), grid, dim3(kKsThreads), 0, s, out, acc, io.add,
                       io.add_stride, io.add_mask, p->dev, p->qp->logn, p->nq, p->np, groups, out_rot, acc_rot, ha);
  else
    hipLaunchKernelGGL((moddown_kernel<B60, KP, false>), grid, dim3(kKsThreads), 0, s, out, acc, io.add,
                       io.add_stride, io.add_mask, p->dev, p->qp->logn, p->nq, p->np, groups, out_rot, acc_rot, ha);
}

constexpr uint64_t kMaxGridY = 65535;

// ModUp of `batch` inputs into ext [batch][dnum][nqp][n] (sigma_h gathered on load).
// grid.y carries batch x digits; a batch whose product exceeds the grid's y range is
// split into chunks.
int ks_modup(const ntt_ks_plan* p, uint64_t* ext, const KsIo& io, uint32_t h, uint64_t batch, hipStream_t s) {
  const uint32_t n = p->qp->n, nqp = p->nq + p->np, dnum = p->dnum;
  const uint32_t tiles = (n + kKsThreads - 1) / kKsThreads;
  // Groups of target primes per coefficient (the Garner digits are recomputed per
  // group): more resident waves for the longer Shoup chains at or above 2^60.
  const uint32_t up_groups = std::max(1u, std::min(p->below60 ? kModUpGroups : kModUpGroupsWide, nqp - p->alpha));
  const uint64_t up_chunk = std::max<uint64_t>(1, kMaxGridY / dnum);
  for (uint64_t b0 = 0; b0 < batch; b0 += up_chunk) {
    const uint64_t nb = std::min(up_chunk, batch - b0);
    KsIo c = io;
    c.src += b0 * io.src_stride;
    const dim3 grid(tiles, (uint32_t)(nb * dnum), up_groups);
    uint64_t* e = ext + b0 * dnum * nqp * n;
    if (p->below60) {
      if (p->alpha <= 8) launch_modup<true, 8>(grid, s, e, c, p, h);
      else launch_modup<true, 16>(grid, s, e, c, p, h);
    } else {
      if (p->alpha <= 8) launch_modup<false, 8>(grid, s, e, c, p, h);
      else launch_modup<false, 16>(grid, s, e, c, p, h);
    }
    if (hipGetLastError() != hipSuccess) return NTT_EDEVICE;
  }
  return NTT_OK;
}

// ModDown of acc [R][batch][2][nqp][n] into out [R][batch][2][nq][n], adding the
// sigma_{h_r} gathered additive inputs selected by io.add_mask (R = num_rot, with
// ha.h[r] the inverse Galois element of rotation r).  One launch covers every
// rotation (grid.z = R x groups).
int ks_moddown(const ntt_ks_plan* p, uint64_t* out, const uint64_t* acc, const KsIo& io, const HoistArgs& ha,
               uint32_t num_rot, uint64_t batch, hipStream_t s) {
  const uint32_t n = p->qp->n, nq = p->nq, nqp = nq + p->np;
  const uint32_t tiles = (n + kKsThreads - 1) / kKsThreads;
  // Groups of output primes recompute the Garner digits over P but add waves: they pay
  // for one ciphertext; several rotations or ciphertexts fill the GPU with one group.
  const uint32_t groups = (uint64_t)num_rot * batch >= 4 ? 1u : std::max(1u, std::min(kModDownGroups, nq));
  const uint64_t out_rot = batch * 2 * nq * n, acc_rot = batch * 2 * nqp * n;
  const uint64_t down_chunk = kMaxGridY / 2;
  for (uint64_t b0 = 0; b0 < batch; b0 += down_chunk) {
    const uint64_t nb = std::min(down_chunk, batch - b0);
    KsIo c = io;
    c.add += b0 * io.add_stride;
    const dim3 grid(tiles, (uint32_t)(nb * 2), num_rot * groups);
    uint64_t* o = out + b0 * 2 * nq * n;
    const uint64_t* a = acc + b0 * 2 * nqp * n;
    if (p->below60) {
      if (p->np <= 8) launch_moddown<true, 8>(grid, s, o, a, c, p, groups, out_rot, acc_rot, ha);
      else launch_moddown<true, 16>(grid, s, o, a, c, p, groups, out_rot, acc_rot, ha);
    } else {
      if (p->np <= 8) launch_moddown<false, 8>(grid, s, o, a, c, p, groups, out_rot, acc_rot, ha);
      else launch_moddown<false, 16>(grid, s, o, a, c, p, groups, out_rot, acc_rot, ha);
    }
    if (hipGetLastError() != hipSuccess) return NTT_EDEVICE;
  }
  return NTT_OK;
}

uint32_t galois_inverse(const ntt_plan* qp, uint64_t g) {
  const uint32_t two_n = 2 * qp->n;
  return (uint32_t)host_invmod(g % two_n, two_n);
}

// The five launches of one key-switch (arguments validated).
int ks_run(const ntt_ks_plan* p, uint64_t* out, const KsIo& io, const uint64_t* ksk, uint64_t galois_elt,
           uint64_t batch, void* workspace, hipStream_t s) {
  const ntt_plan* qp = p->qp;
  const uint32_t n = qp->n, nqp = p->nq + p->np, dnum = p->dnum;
  DeviceGuard g(qp->device);
  if (!g.ok) return NTT_EDEVICE;
  uint64_t* ext = (uint64_t*)workspace;
  uint64_t* acc = ext + batch * (uint64_t)dnum * nqp * n;
  const uint32_t h = galois_inverse(qp, galois_elt);
  int rc = ks_modup(p, ext, io, h, batch, s);
  if (rc) return rc;
  if (ks_middle_supported(qp, dnum, p->mac_chunk)) {  // forward NTT, key product, inverse NTT
    if (launch_ks_middle(qp, acc, ext, ksk, batch, nqp, dnum, s) != hipSuccess) return NTT_EDEVICE;
    HoistArgs ha{};
    ha.h[0] = h;
    return ks_moddown(p, out, acc, io, ha, 1, batch, s);
  }
  if (launch_ntt(qp, ext, batch * dnum, 0, nqp, false, s) != hipSuccess) return NTT_EDEVICE;
  if (intt_mac_supported(qp)) {  // key product fused into the inverse transform's first pass
    if (launch_intt_mac(qp, acc, ext, ksk, batch, nqp, dnum, p->mac_chunk, s) != hipSuccess) return NTT_EDEVICE;
    HoistArgs ha{};
    ha.h[0] = h;
    return ks_moddown(p, out, acc, io, ha, 1, batch, s);
  }
  const uint64_t pairs = (uint64_t)nqp * n / 2;
  for (uint64_t b0 = 0; b0 < batch; b0 += kMaxGridY) {
    const uint64_t nb = std::min(kMaxGridY, batch - b0);
    hipLaunchKernelGGL(mac_kernel, dim3((uint32_t)((pairs + kKsThreads - 1) / kKsThreads), (uint32_t)nb),
                       dim3(kKsThreads), 0, s, acc + b0 * 2 * nqp * n, ext + b0 * dnum * nqp * n, ksk, qp->d_mods,
                       qp->logn, nqp, dnum, p->mac_chunk, pairs);
    if (hipGetLastError() != hipSuccess) return NTT_EDEVICE;
  }
  if (launch_ntt(qp, acc, batch * 2, 0, nqp, true, s) != hipSuccess) return NTT_EDEVICE;
  HoistArgs ha{};
  ha.h[0] = h;
  return ks_moddown(p, out, acc, io, ha, 1, batch, s);
}
}  // namespace

extern "C" int keyswitch(const ntt_ks_plan* p, uint64_t* out, const uint64_t* ct, const uint64_t* ksk,
                         uint64_t galois_elt, uint64_t batch, void* workspace, size_t workspace_bytes, void* stream) {
  if (!p) return NTT_EINVAL;
  const uint32_t n = p->qp->n;
  const uint64_t plane = (uint64_t)p->nq * n;
  if (!(galois_elt & 1) || galois_elt >= 2ull * n) return NTT_EINVAL;
  if (batch == 0) return NTT_OK;
  const KsIo io{ct ? ct + plane : nullptr, 2 * plane, ct, 2 * plane, 1u, batch * 2 * plane * 8, ct};
  int rc = ks_check(p, out, io, ksk, batch, workspace, workspace_bytes);
  if (rc) return rc;
  if ((rc = ks_debug_inputs(p, ct, 2 * batch, ksk, p->dnum * 2, (hipStream_t)stream))) return rc;
  return ks_run(p, out, io, ksk, galois_elt, batch, workspace, (hipStream_t)stream);
}

extern "C" int relinearize(const ntt_ks_plan* p, uint64_t* out, const uint64_t* d, const uint64_t* rlk,
                           uint64_t batch, void* workspace, size_t workspace_bytes, void* stream) {
  if (!p) return NTT_EINVAL;
  const uint64_t plane = (uint64_t)p->nq * p->qp->n;
  if (batch == 0) return NTT_OK;
  // decompose d2, add (d0, d1); no automorphism (g = 1)
  const KsIo io{d ? d + 2 * plane : nullptr, 3 * plane, d, 3 * plane, 3u, batch * 3 * plane * 8, d};
  int rc = ks_check(p, out, io, rlk, batch, workspace, workspace_bytes);
  if (rc) return rc;
  if ((rc = ks_debug_inputs(p, d, 3 * batch, rlk, p->dnum * 2, (hipStream_t)stream))) return rc;
  return ks_run(p, out, io, rlk, 1, batch, workspace, (hipStream_t)stream);
}

extern "C" int keyswitch_hoisted_workspace_size(const ntt_ks_plan* p, uint32_t num_rot, uint64_t batch,
                                               size_t* bytes) {
  if (!p || !bytes || num_rot == 0) return NTT_EINVAL;
  if (batch > 4096 || num_rot > kMaxHoisted) return NTT_EUNSUPPORTED;
  const uint64_t qplane = (uint64_t)(p->nq + p->np) * p->qp->n, plane = (uint64_t)p->nq * p->qp->n;
  *bytes = (size_t)(batch * ((p->dnum + 2ull * num_rot) * qplane + plane) * 8);
  return NTT_OK;
}

extern "C" int keyswitch_hoisted(const ntt_ks_plan* p, uint64_t* out, const uint64_t* ct, const uint64_t* ksk,
                                 const uint64_t* galois_elts, uint32_t num_rot, uint64_t batch, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (!p || !galois_elts || num_rot == 0) return NTT_EINVAL;
  const ntt_plan* qp = p->qp;
  const uint32_t n = qp->n, nq = p->nq, nqp = nq + p->np, dnum = p->dnum;
  if (num_rot > kMaxHoisted || batch > 4096) return NTT_EUNSUPPORTED;
  if (dnum > 16) return NTT_EUNSUPPORTED;  // the digits of one segment are staged in LDS
  for (uint32_t r = 0; r < num_rot; ++r)
    if (!(galois_elts[r] & 1) || galois_elts[r] >= 2ull * n) return NTT_EINVAL;
  if (batch == 0) return NTT_OK;
  if (!out || !ct || !ksk || !workspace) return NTT_EINVAL;
  if (((uintptr_t)out | (uintptr_t)ct | (uintptr_t)ksk) & 15u) return NTT_EINVAL;
  if ((uintptr_t)workspace & 255u) return NTT_EINVAL;
  const uint64_t plane = (uint64_t)nq * n, qplane = (uint64_t)nqp * n;
  const uint64_t need = batch * ((dnum + 2ull * num_rot) * qplane + plane) * 8;
  if (workspace_bytes < need) return NTT_EINVAL;
  const uint64_t ct_bytes = batch * 2 * plane * 8, out_bytes = num_rot * ct_bytes;
  const uint64_t ksk_bytes = (uint64_t)num_rot * dnum * 2 * qplane * 8;
  if (ranges_overlap(out, out_bytes, ct, ct_bytes) || ranges_overlap(out, out_bytes, ksk, ksk_bytes) ||
      ranges_overlap(out, out_bytes, workspace, need) || ranges_overlap(workspace, need, ct, ct_bytes) ||
      ranges_overlap(workspace, need, ksk, ksk_bytes))
    return NTT_EOVERLAP;

  int rc = ks_debug_inputs(p, ct, 2 * batch, ksk, (uint64_t)num_rot * dnum * 2, (hipStream_t)stream);
  if (rc) return rc;
  DeviceGuard g(qp->device);
  if (!g.ok) return NTT_EDEVICE;
  hipStream_t s = (hipStream_t)stream;
  HoistArgs ha{};
  for (uint32_t r = 0; r < num_rot; ++r) {
    ha.g[r] = (uint32_t)galois_elts[r];
    ha.h[r] = galois_inverse(qp, galois_elts[r]);
  }
  uint64_t* ext = (uint64_t*)workspace;
  uint64_t* acc = ext + batch * (uint64_t)dnum * qplane;
  uint64_t* c0hat = acc + batch * 2ull * num_rot * qplane;  // [batch][nq][n]
  const KsIo io{ct + plane, 2 * plane, ct, 2 * plane, 1u, ct_bytes, ct};
  rc = ks_modup(p, ext, io, 1, batch, s);  // no automorphism: the digits are shared
  if (rc) return rc;
  if (launch_ntt(qp, ext, batch * dnum, 0, nqp, false, s) != hipSuccess) return NTT_EDEVICE;
  if (intt_mac_supported(qp)) {  // key products fused into the inverse transform's first pass
    // Every rotation adds sigma_g(c0) to its output: as P sigma_g(c0), a slot permutation
    // of P NTT(c0), it joins the key product, and ModDown runs without a gather.
    const bool fold = dnum <= 4 && p->mac_chunk_max > dnum;
    if (fold)
      for (uint64_t b = 0; b < batch; ++b)
        if (launch_ntt_galois(qp, c0hat + b * plane, ct + b * 2 * plane, 1, 1, 0, nq, s) != hipSuccess)
          return NTT_EDEVICE;
    if (launch_intt_mac_hoisted(qp, acc, ext, ksk, batch, num_rot, nqp, dnum,
                                fold ? p->mac_chunk_max : p->mac_chunk, ha, fold ? c0hat : nullptr, p->dev.p_r64,
                                nq, s) != hipSuccess)
      return NTT_EDEVICE;
    KsIo down = io;
    if (fold) down.add_mask = 0;
    return ks_moddown(p, out, acc, down, ha, num_rot, batch, s);
  }
  const uint32_t seglog = std::min(qp->logn, 9u);
  const dim3 grid((nqp << (qp->logn - seglog)), (uint32_t)batch);
  hipLaunchKernelGGL(mac_hoisted_kernel, grid, dim3(kKsThreads), (size_t)dnum * (8u << seglog), s, acc, ext, ksk,
                     qp->d_mods, qp->logn, seglog, nqp, dnum, p->mac_chunk, num_rot, (uint32_t)batch, ha);
  if (hipGetLastError() != hipSuccess) return NTT_EDEVICE;
  if (launch_ntt(qp, acc, batch * 2 * num_rot, 0, nqp, true, s) != hipSuccess) return NTT_EDEVICE;
  return ks_moddown(p, out, acc, io, ha, num_rot, batch, s);
}

extern "C" void keyswitch_plan_destroy(ntt_ks_plan* p) {
  if (!p) return;
  if (p->d_const) {
    DeviceGuard g(p->qp->device);
    (void)hipFree(p->d_const);
  }
  delete p;
}

// ---- ModRaise plan ----------------------------------------------------------------------

struct ntt_mr_plan {
  const ntt_plan* plan = nullptr;
  uint32_t from = 0, to = 0;
  bool below60 = false;
  void* d_const = nullptr;
  const uint64_t* moduli = nullptr;  // [to]
  const Tw* garner = nullptr;        // [K][K] over the first `from` primes
  const Tw* eval = nullptr;          // [to][K]
};

extern "C" int modraise_plan_create(ntt_mr_plan** out, const ntt_plan* plan, uint32_t from, uint32_t to) {
  if (!out) return NTT_EINVAL;
  *out = nullptr;
  if (!plan) return NTT_EINVAL;
  if (plan->device < 0) return NTT_EDEVICE;
  if (from == 0 || to <= from || to > plan->num_primes) return NTT_EINVAL;
  if (from > (uint32_t)kMaxDigitPrimes) return NTT_EUNSUPPORTED;
  const uint32_t K = (uint32_t)kMaxDigitPrimes;
  const uint64_t* m = plan->primes.data();
  std::vector<Tw> gar((size_t)K * K, Tw{0, 0}), ev((size_t)to * K, Tw{0, 0});
  garner_table(m, from, K, gar.data());
  for (uint32_t t = 0; t < to; ++t) eval_table(m, from, m[t], ev.data() + (size_t)t * K);
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t sz_m = (size_t)to * 8, sz_g = gar.size() * sizeof(Tw), sz_e = ev.size() * sizeof(Tw);
  const size_t total = al(sz_m) + al(sz_g) + al(sz_e);
  std::vector<uint8_t> blob(total, 0);
  memcpy(blob.data(), m, sz_m);
  memcpy(blob.data() + al(sz_m), gar.data(), sz_g);
  memcpy(blob.data() + al(sz_m) + al(sz_g), ev.data(), sz_e);
  ntt_mr_plan* p = new (std::nothrow) ntt_mr_plan;
  if (!p) return NTT_ENOMEM;
  {
    DeviceGuard g(plan->device);
    if (!g.ok) {
      delete p;
      return NTT_EDEVICE;
    }
    if (hipMalloc(&p->d_const, total) != hipSuccess) {
      delete p;
      return NTT_ENOMEM;
    }
    if (hipMemcpy(p->d_const, blob.data(), total, hipMemcpyHostToDevice) != hipSuccess) {
      (void)hipFree(p->d_const);
      delete p;
      return NTT_EDEVICE;
    }
  }
  uint8_t* base = (uint8_t*)p->d_const;
  p->plan = plan;
  p->from = from;
  p->to = to;
  p->below60 = range_below60(plan, 0, to);
  p->moduli = (const uint64_t*)base;
  p->garner = (const Tw*)(base + al(sz_m));
  p->eval = (const Tw*)(base + al(sz_m) + al(sz_g));
  *out = p;
  return NTT_OK;
}

extern "C" int modraise(const ntt_mr_plan* p, uint64_t* out, const uint64_t* in, uint64_t batch, void* stream) {
  if (!p) return NTT_EINVAL;
  const ntt_plan* plan = p->plan;
  const uint32_t n = plan->n;
  if (batch > (1ull << 36) / ((uint64_t)p->to * n)) return NTT_EUNSUPPORTED;
  if (batch == 0) return NTT_OK;
  if (!out || !in || (((uintptr_t)out | (uintptr_t)in) & 15u)) return NTT_EINVAL;
  if (ranges_overlap(out, batch * p->to * n * 8, in, batch * p->from * n * 8)) return NTT_EOVERLAP;
  const int rc = debug_check_inputs(plan, in, batch, 0, p->from, (hipStream_t)stream);
  if (rc) return rc;
  DeviceGuard g(plan->device);
  if (!g.ok) return NTT_EDEVICE;
  hipStream_t s = (hipStream_t)stream;
  const uint32_t tiles = (n + kKsThreads - 1) / kKsThreads;
  const uint32_t others = p->to - p->from;
  for (uint64_t b0 = 0; b0 < batch; b0 += kMaxGridY) {
    const uint64_t nb = std::min(kMaxGridY, batch - b0);
    // enough blocks to fill the chip; the Garner digits are recomputed per group
    const uint64_t base = (uint64_t)tiles * nb;
    const uint32_t groups = (uint32_t)std::max<uint64_t>(1, std::min<uint64_t>(others, (2048 + base - 1) / base));
    const dim3 grid(tiles, (uint32_t)nb, groups);
    uint64_t* o = out + b0 * p->to * n;
    const uint64_t* x = in + b0 * p->from * n;
    if (p->below60) {
      if (p->from <= 4)
        hipLaunchKernelGGL((modraise_kernel<true, 4>), grid, dim3(kKsThreads), 0, s, o, x, p->moduli, p->garner,
                           p->eval, plan->logn, p->from, p->to);
      else
        hipLaunchKernelGGL((modraise_kernel<true, 16>), grid, dim3(kKsThreads), 0, s, o, x, p->moduli, p->garner,
                           p->eval, plan->logn, p->from, p->to);
    } else {
      if (p->from <= 4)
        hipLaunchKernelGGL((modraise_kernel<false, 4>), grid, dim3(kKsThreads), 0, s, o, x, p->moduli, p->garner,
                           p->eval, plan->logn, p->from, p->to);
      else
        hipLaunchKernelGGL((modraise_kernel<false, 16>), grid, dim3(kKsThreads), 0, s, o, x, p->moduli, p->garner,
                           p->eval, plan->logn, p->from, p->to);
    }
    if (hipGetLastError() != hipSuccess) return NTT_EDEVICE;
  }
  return NTT_OK;
}

extern "C" void modraise_plan_destroy(ntt_mr_plan* p) {
  if (!p) return;
  if (p->d_const) {
    DeviceGuard g(p->plan->device);
    (void)hipFree(p->d_const);
  }
  delete p;
}
