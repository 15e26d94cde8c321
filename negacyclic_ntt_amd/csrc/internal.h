// Internal declarations shared by the library's translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "modarith.h"
#include "negacyclic_ntt.h"

namespace nntt {

// Per-prime constants, device resident (one entry per plan prime).
struct ModInfo {
  uint64_t q;
  uint64_t n_inv, n_inv_shoup;  // n^-1 mod q and floor(n^-1 * 2^64 / q)
  uint64_t n_inv_shoup60;       // floor(n^-1 * 2^62 / q) (primes below 2^60)
  uint32_t n_inv32, n_inv_shoup32;  // narrow (q < 2^30) Shoup pair, else 0
  // w1n = psi^-brv(1) n^-1 mod q: the inverse network's last-stage twiddle with the
  // final scaling folded in, and its Shoup companions (2^64, 2^62, 2^32 scaled).
  uint64_t w1n, w1n_shoup, w1n_shoup60;
  uint32_t w1n32, w1n_shoup32;
  Barrett br;
  uint64_t mont_ninv;  // -q^-1 mod 2^64 (Montgomery reduction with R = 2^64)
  uint64_t r64, r64_shoup;  // 2^64 mod q and floor(r64 2^64 / q): undoes a Montgomery reduction
};

// Constants to divide by prime k and express the quotient modulo prime l < k (rescale).
// Stored as a triangle: entry k (k - 1) / 2 + l.
struct RescaleC {
  uint64_t inv, inv_shoup;  // q_k^-1 mod q_l and floor(inv * 2^64 / q_l)
  uint64_t m;               // q_l * ceil(q_k / q_l): a multiple of q_l that is >= q_k
  uint64_t half;            // floor(q_k / 2) mod q_l
};
__host__ __device__ inline size_t rescale_index(uint32_t k, uint32_t l) { return (size_t)k * (k - 1) / 2 + l; }

constexpr uint32_t kMaxLogN = 16;

// Device twiddle layout for the two-pass split (n = 2^15, 2^16: rows of N2 = 2^8, the
// row transform in two radix-16 passes).  The row transform's last pass (row stages
// 4..7) reads, for row r and set u (0..15) at row stage 4 + v, the 2^v entries
// ((N1 + r) 2^4 + u) 2^v + j.  Stored instead at (N1 + r) 2^(4 + v) + j 2^4 + u, so that
// for each (v, j) the 16 sets of a row read 16 consecutive entries: each stage block
// [2^s, 2^(s+1)) is permuted within each row's sub-block only.  Host copies returned
// by ntt_plan_get_tables keep the plain order.
constexpr uint32_t kPermMinLogN = 15, kPermRowLog = 8, kPermRowS0 = 4;
__host__ __device__ constexpr bool row_tw_permuted(uint32_t logn) { return logn >= kPermMinLogN; }

// The NTT-domain automorphism in bit-reversed slot order: out[k] = in[slot(k)] with
// 2 brv(slot) + 1 = (2 brv(k) + 1) g mod 2n, i.e. brv(slot) = g brv(k) + (g - 1) / 2
// mod n.  It maps every aligned segment of 2^m slots onto an aligned segment: the
// low log n - m bits of g brv(k) + c depend only on those of brv(k), which are the
// reversed high bits of k, fixed inside the segment.
__device__ __forceinline__ uint32_t ntt_slot(uint32_t k, uint32_t g, uint32_t logn) {
  const uint32_t K = __brev(k) >> (32 - logn);
  const uint32_t P = (uint32_t)(((uint64_t)K * g + (g >> 1)) & ((1u << logn) - 1));
  return __brev(P) >> (32 - logn);
}

// Galois elements of a hoisted key-switch (and their inverses mod 2n), passed by value.
constexpr uint32_t kMaxHoisted = 64;
struct HoistArgs {
  uint32_t g[kMaxHoisted];
  uint32_t h[kMaxHoisted];
};
constexpr uint32_t kMaxPrimes = 4096;

}  // namespace nntt

struct ntt_plan {
  uint32_t n = 0, logn = 0, num_primes = 0;
  int device = -1;
  std::vector<uint64_t> primes, psis;
  std::vector<uint8_t> narrow;                   // 1 if q < 2^30
  std::vector<uint8_t> below60;                  // 1 if q < 2^60
  std::vector<uint64_t> h_fwd, h_fwd_sh, h_inv, h_inv_sh;  // host tables [L][n]
  std::vector<nntt::ModInfo> h_mods;
  // device copies
  nntt::Wide::Tw* d_fwd = nullptr;    // [L][n] {psi^brv(k), shoup}
  nntt::Wide::Tw* d_inv = nullptr;    // [L][n] {psi^-brv(k), shoup}
  nntt::Wide60::Tw* d_fwd60 = nullptr;  // [L][n] {w, floor(w * 2^62 / q)}, zero for q >= 2^60
  nntt::Wide60::Tw* d_inv60 = nullptr;
  nntt::Narrow::Tw* d_fwd32 = nullptr;  // [L][n], entries of wide primes are zero
  nntt::Narrow::Tw* d_inv32 = nullptr;
  nntt::ModInfo* d_mods = nullptr;    // [L]
  nntt::RescaleC* d_rescale = nullptr;  // triangle over the plan's primes, L (L - 1) / 2 entries
  unsigned long long* d_check = nullptr;  // one counter for the debug input checks
};

namespace nntt {

// Host helpers (plan.cpp)
uint64_t host_mulmod(uint64_t a, uint64_t b, uint64_t q);
uint64_t host_powmod(uint64_t b, uint64_t e, uint64_t q);
uint64_t host_invmod(uint64_t a, uint64_t q);
bool host_is_prime(uint64_t n);
Barrett host_barrett(uint64_t q);

// Blocks are dispatched round-robin over the 8 XCDs of an MI355X: hardware block b runs
// on XCD b % 8.  xcd_local_block maps b to a logical block so that each XCD works on one
// contiguous range of logical blocks (and hence of the data), keeping its L2 working set
// local.  Identity for the tail that does not fill all eight.
__device__ __forceinline__ uint32_t xcd_local_block(uint32_t b, uint32_t nblocks) {
  constexpr uint32_t kXcd = 8;
  const uint32_t full = nblocks - nblocks % kXcd;
  if (b >= full) return b;
  return (b % kXcd) * (full / kXcd) + b / kXcd;
}

// RAII device selection: makes `dev` current and restores the previous device.
struct DeviceGuard {
  int prev = -1;
  bool ok = false;
  explicit DeviceGuard(int dev);
  ~DeviceGuard();
};

// Threads of one launch: a dispatch packet holds at most 2^32 - 1 work-items per
// grid dimension.  max_launch_threads() is this cap, or the smaller one set through
// ntt_set_max_launch_threads (capi.cpp).
// The default cap leaves room for the rounding up of a launch to whole workgroups.
constexpr uint64_t kMaxLaunchThreads = 0xffff0000ull;
uint64_t max_launch_threads();
// Items (polynomials, ciphertexts) per launch when each needs `threads_per_item`
// threads; 0 when one item alone exceeds the cap.
inline uint64_t items_per_launch(uint64_t threads_per_item) {
  return threads_per_item ? max_launch_threads() / threads_per_item : 0;
}

// Launchers (ntt.hip). Arguments already validated. Return the launch status
// (hipErrorInvalidConfiguration when one polynomial exceeds the launch cap).
hipError_t launch_ntt(const ntt_plan* p, uint64_t* data, uint64_t batch, uint32_t limb_begin, uint32_t num_limbs,
                      bool inverse, hipStream_t s);
hipError_t launch_ntt_galois(const ntt_plan* p, uint64_t* out, const uint64_t* in, uint64_t g, uint64_t batch,
                             uint32_t limb_begin, uint32_t num_limbs, hipStream_t s);
// Key product fused into the inverse transform (two-pass sizes, n >= 2^15): acc
// [batch][2][nqp][n] = INTT( sum_j ext[b][j] * ksk[j][c] ) with the digits ext in
// Montgomery form (times 2^64) and `chunk` products summed per reduction.
bool intt_mac_supported(const ntt_plan* p);
hipError_t launch_intt_mac(const ntt_plan* p, uint64_t* acc, const uint64_t* ext, const uint64_t* ksk, uint64_t batch,
                           uint32_t nqp, uint32_t dnum, uint32_t chunk, hipStream_t s);
// The whole middle of a key-switch for the two-pass sizes (n >= 2^15, 1 <= dnum <= 4 and
// one reduction for the dnum products, chunk >= dnum): forward NTT of the digits ext
// [batch][dnum][nqp][n] (Montgomery form; overwritten), key product and inverse NTT
// into acc [batch][2][nqp][n].  The NTT-domain digits stay in LDS between the forward
// row pass and the key product.
bool ks_middle_supported(const ntt_plan* p, uint32_t dnum, uint32_t chunk);
hipError_t launch_ks_middle(const ntt_plan* p, uint64_t* acc, uint64_t* ext, const uint64_t* ksk, uint64_t batch,
                            uint32_t nqp, uint32_t dnum, hipStream_t s);
// The same for hoisted rotations: acc [num_rot][batch][2][nqp][n] from the shared digits
// gathered through each rotation's slot permutation, keys [num_rot][dnum][2][nqp][n].
// c0hat (nullable): NTT(c0) [batch][nq][n]; with it component 0 also sums P * NTT(c0)
// through the rotation's slot permutation (pr64[t] = P 2^64 mod q_t, t < nq), which then
// takes chunk > dnum (one more product per reduction).
hipError_t launch_intt_mac_hoisted(const ntt_plan* p, uint64_t* acc, const uint64_t* ext, const uint64_t* ksk,
                                   uint64_t batch, uint32_t num_rot, uint32_t nqp, uint32_t dnum, uint32_t chunk,
                                   const HoistArgs& ha, const uint64_t* c0hat, const uint64_t* pr64, uint32_t nq,
                                   hipStream_t s);
// True when every prime in [limb_begin, limb_begin + num_limbs) is below 2^30.
bool range_is_narrow(const ntt_plan* p, uint32_t limb_begin, uint32_t num_limbs);
// True when every prime in the range is below 2^60.
bool range_below60(const ntt_plan* p, uint32_t limb_begin, uint32_t num_limbs);

// Coefficient-domain ciphertext product (ntt.hip), n <= 2^12: out [batch][3][L][n] =
// INTT(tensor(NTT(a), NTT(b))) for a, b [batch][2][L][n], one launch.
bool chain_supported(const ntt_plan* p);
hipError_t launch_ct_tensor_coeff(const ntt_plan* p, uint64_t* out, const uint64_t* a, const uint64_t* b,
                                  uint64_t batch, uint32_t limb_begin, uint32_t num_limbs, hipStream_t s);

// HIP device of a key-switch plan (keyswitch.hip).
int ks_plan_device(const ntt_ks_plan* p);

// Element-wise launchers (elementwise.hip).
hipError_t launch_pointwise(const ntt_plan* p, uint64_t* out, const uint64_t* a, const uint64_t* b, uint64_t batch,
                            uint32_t limb_begin, uint32_t num_limbs, hipStream_t s);
hipError_t launch_tensor(const ntt_plan* p, uint64_t* out, const uint64_t* a, const uint64_t* b, uint64_t batch,
                         uint32_t limb_begin, uint32_t num_limbs, hipStream_t s);
hipError_t launch_automorph(const ntt_plan* p, uint64_t* out, const uint64_t* in, uint64_t g, int domain,
                            uint64_t batch, uint32_t limb_begin, uint32_t num_limbs, hipStream_t s);
// Adds the number of residues >= their prime in data [rows][num_limbs][n] to *count.
hipError_t launch_count_noncanonical(const ntt_plan* p, const uint64_t* data, uint64_t rows, uint32_t limb_begin,
                                     uint32_t num_limbs, unsigned long long* count, hipStream_t s);
hipError_t launch_zero_counter(unsigned long long* count, hipStream_t s);
// Debug input checks (capi.cpp): when enabled, counts the non-canonical residues of an
// input [rows][num_limbs][n] and waits for the result: NTT_EINVAL if any, else NTT_OK.
// Disabled: NTT_OK without touching the device.
int debug_check_inputs(const ntt_plan* p, const uint64_t* data, uint64_t rows, uint32_t limb_begin,
                       uint32_t num_limbs, hipStream_t s);
// in: [batch][num_limbs][n] over primes [limb_begin, limb_begin + num_limbs); out: [batch][num_limbs - 1][n].
hipError_t launch_rescale(const ntt_plan* p, uint64_t* out, const uint64_t* in, uint64_t batch, uint32_t limb_begin,
                          uint32_t num_limbs, bool nearest, hipStream_t s);

}  // namespace nntt
