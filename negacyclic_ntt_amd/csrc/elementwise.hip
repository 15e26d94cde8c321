// Element-wise kernels: pointwise products, the ciphertext tensor product, the
// Galois automorphisms, rescale and the non-canonical count.  All are bound by
// memory traffic, so each thread moves 16-byte vectors (the coefficient automorphism:
// one gathered 16-byte pair, two 8-byte stores) and the arithmetic (Barrett and Shoup
// products) is off the critical path.
//
// FHElium ("Eager, Compile, and native execution", section "CUDA execution")
// maps kernel grids onto the tensor axes limb x coefficient tile x batch; here the
// [batch][limb][n] tensor is treated as one flat array whose row r has limb
// r % num_limbs, which covers the same axes with a 1-D grid (split into launches of
// whole polynomials when it would exceed the launch cap).
#include <algorithm>

#include "internal.h"

namespace nntt {
namespace {

constexpr int kThreads = 256;

// Streaming 16-byte accesses: every residue is touched once, so loads and stores are
// marked non-temporal (they bypass reuse-oriented cache allocation).
typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u64x2 ld_stream(const uint64_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u64x2*>(p));
}
__device__ __forceinline__ void st_stream(uint64_t* p, u64x2 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u64x2*>(p));
}

__global__ __launch_bounds__(kThreads) void pointwise_kernel(uint64_t* __restrict__ out,
                                                             const uint64_t* __restrict__ a,
                                                             const uint64_t* __restrict__ b,
                                                             const ModInfo* __restrict__ mods, uint32_t logn,
                                                             uint32_t num_limbs, uint32_t limb_begin,
                                                             uint64_t pairs) {
  const uint64_t p = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
  if (p >= pairs) return;
  const uint64_t e = 2 * p;
  const Barrett br = mods[limb_begin + (uint32_t)((e >> logn) % num_limbs)].br;
  const u64x2 x = ld_stream(a + e);
  const u64x2 y = ld_stream(b + e);
  u64x2 z;
  z.x = barrett_mul(x.x, y.x, br);
  z.y = barrett_mul(x.y, y.y, br);
  st_stream(out + e, z);
}

// a, b: [batch][2][L][n]; out: [batch][3][L][n].
__global__ __launch_bounds__(kThreads) void tensor_kernel(uint64_t* __restrict__ out,
                                                          const uint64_t* __restrict__ a,
                                                          const uint64_t* __restrict__ b,
                                                          const ModInfo* __restrict__ mods, uint32_t logn,
                                                          uint32_t num_limbs, uint32_t limb_begin,
                                                          uint64_t pairs) {
  const uint64_t p = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
  if (p >= pairs) return;
  const uint64_t plane = (uint64_t)num_limbs << logn;  // elements per component
  const uint64_t e = 2 * p;                            // flat index in [batch][L][n]
  const uint64_t bi = e / plane, off = e % plane;
  const ModInfo& mi = mods[limb_begin + (uint32_t)(off >> logn)];
  const Barrett br = mi.br;
  const uint64_t q = br.q;
  const uint64_t* a0 = a + bi * 2 * plane + off;
  const uint64_t* b0 = b + bi * 2 * plane + off;
  uint64_t* d0 = out + bi * 3 * plane + off;
  const u64x2 x0 = ld_stream(a0);
  const u64x2 x1 = ld_stream(a0 + plane);
  const u64x2 y0 = ld_stream(b0);
  const u64x2 y1 = ld_stream(b0 + plane);
  u64x2 r0, r1, r2;
  r0.x = barrett_mul(x0.x, y0.x, br);
  r0.y = barrett_mul(x0.y, y0.y, br);
  // d1 = a0 b1 + a1 b0: the exact 128-bit sum (< 2 q^2 < q 2^64) reduced once by
  // Montgomery (which divides by 2^64), then one Shoup product by 2^64 mod q.
  {
    const Wide::Tw r64{mi.r64, mi.r64_shoup};
    Acc128 s0{0, 0}, s1{0, 0};
    mac128(s0, x0.x, y1.x);
    mac128(s0, x1.x, y0.x);
    mac128(s1, x0.y, y1.y);
    mac128(s1, x1.y, y0.y);
    r1.x = csub(Wide::mul(redc(s0, q, mi.mont_ninv), r64, q), q);
    r1.y = csub(Wide::mul(redc(s1, q, mi.mont_ninv), r64, q), q);
  }
  r2.x = barrett_mul(x1.x, y1.x, br);
  r2.y = barrett_mul(x1.y, y1.y, br);
  st_stream(d0, r0);
  st_stream(d0 + plane, r1);
  st_stream(d0 + 2 * plane, r2);
}

// Coefficient domain: out[e] = in[i] if i < n else -in[i - n], i = e * h mod 2n,
// h = g^-1 mod 2n (the inverse of the scatter i -> i g).  Gather form: writes are
// coalesced, reads hit L2 thanks to the XCD-local block order.
__global__ __launch_bounds__(kThreads) void automorph_coeff_kernel(uint64_t* __restrict__ out,
                                                                   const uint64_t* __restrict__ in,
                                                                   const ModInfo* __restrict__ mods,
                                                                   uint32_t logn, uint32_t h,
                                                                   uint32_t num_limbs, uint32_t limb_begin,
                                                                   uint64_t total) {
  const uint32_t lb = xcd_local_block(blockIdx.x, gridDim.x);
  const uint64_t idx = (uint64_t)lb * kThreads + threadIdx.x;
  if (idx >= total) return;
  const uint32_t n = 1u << logn, mask2n = 2 * n - 1;
  const uint64_t row = idx >> logn;
  const uint32_t e = (uint32_t)(idx & (n - 1));
  const uint32_t i = (uint32_t)(((uint64_t)e * h) & mask2n);
  const uint64_t q = mods[limb_begin + (uint32_t)(row % num_limbs)].q;
  const uint64_t* src = in + (row << logn);
  uint64_t v;
  if (i < n)
    v = src[i];
  else
    v = neg_mod(src[i - n], q);
  __builtin_nontemporal_store(v, out + idx);
}

// The same gather with P consecutive outputs per thread (P independent loads in flight,
// one P x 8-byte store).  Launched only when the total is a multiple of P x threads.
template <uint32_t P>
__global__ __launch_bounds__(kThreads) void automorph_coeff_multi_kernel(uint64_t* __restrict__ out,
                                                                         const uint64_t* __restrict__ in,
                                                                         const ModInfo* __restrict__ mods,
                                                                         uint32_t logn, uint32_t h,
                                                                         uint32_t num_limbs, uint32_t limb_begin,
                                                                         uint64_t groups) {
  const uint32_t lb = xcd_local_block(blockIdx.x, gridDim.x);
  const uint64_t gi = (uint64_t)lb * kThreads + threadIdx.x;
  if (gi >= groups) return;
  const uint32_t n = 1u << logn, mask2n = 2 * n - 1;
  const uint64_t idx = gi * P, row = idx >> logn;
  const uint32_t e = (uint32_t)(idx & (n - 1));
  const uint64_t q = mods[limb_begin + (uint32_t)(row % num_limbs)].q;
  const uint64_t* src = in + (row << logn);
  uint64_t v[P];
#pragma unroll
  for (uint32_t k = 0; k < P; ++k) {
    const uint32_t i = (uint32_t)(((uint64_t)(e + k) * h) & mask2n);
    const uint64_t a = src[i & (n - 1)];
    v[k] = i < n ? a : neg_mod(a, q);
  }
#pragma unroll
  for (uint32_t k = 0; k < P; k += 2) st_stream(out + idx + k, u64x2{v[k], v[k + 1]});
}

// Pair form of the same gather.  For an even output e, i = e h mod 2n is even, so the
// input pair (i, i + 1) of the extended sequence in_ext = (in, -in) is one aligned
// 16-byte load.  Its second element belongs to the output o = e + g mod 2n (since
// (e + g) h = i + 1): out[o mod n], negated once more when o >= n (n h = n mod 2n).
// As e runs over the even outputs, o mod n runs over the odd ones once each.  A
// thread therefore reads one pair and writes two outputs: half the gather requests
// of the per-element form, at the price of stores that fill half a line each (the
// other half is the partner of another thread of the same limb, on the same XCD).
// P pairs per thread; a block covers P * kThreads consecutive even outputs of one
// row, so launched only when n / 2 is a multiple of that.  The stores are plain, so
// that the two halves of a line meet in L2 (non-temporal stores: +35% on MI355X).
template <uint32_t P>
__global__ __launch_bounds__(kThreads) void automorph_coeff_pair_kernel(uint64_t* __restrict__ out,
                                                                        const uint64_t* __restrict__ in,
                                                                        const ModInfo* __restrict__ mods,
                                                                        uint32_t logn, uint32_t g, uint32_t h,
                                                                        uint32_t num_limbs, uint32_t limb_begin,
                                                                        uint32_t blocks_per_row) {
  const uint32_t lb = xcd_local_block(blockIdx.x, gridDim.x);
  const uint32_t n = 1u << logn, mask2n = 2 * n - 1;
  const uint64_t row = lb / blocks_per_row;
  const uint32_t pair0 = (lb % blocks_per_row) * (P * kThreads) + threadIdx.x;
  const uint64_t q = mods[limb_begin + (uint32_t)(row % num_limbs)].q;
  const uint64_t* src = in + (row << logn);
  uint64_t* dst = out + (row << logn);
  u64x2 v[P];
  uint32_t e[P], i[P];
#pragma unroll
  for (uint32_t k = 0; k < P; ++k) {
    e[k] = 2 * (pair0 + k * kThreads);
    i[k] = (uint32_t)(((uint64_t)e[k] * h) & mask2n);
    v[k] = *reinterpret_cast<const u64x2*>(src + (i[k] & (n - 1)));
  }
#pragma unroll
  for (uint32_t k = 0; k < P; ++k) {
    const bool neg0 = i[k] >= n;
    const uint32_t o = (e[k] + g) & mask2n;
    const bool neg1 = neg0 != (o >= n);
    dst[e[k]] = neg0 ? neg_mod(v[k].x, q) : v[k].x;
    dst[o & (n - 1)] = neg1 ? neg_mod(v[k].y, q) : v[k].y;
  }
}

// NTT domain (bit-reversed slots): out[k] = in[p(k)], 2 brv(p) + 1 = (2 brv(k) + 1) g mod 2n.
__global__ __launch_bounds__(kThreads) void automorph_ntt_kernel(uint64_t* __restrict__ out,
                                                                 const uint64_t* __restrict__ in, uint32_t logn,
                                                                 uint32_t g, uint64_t total) {
  const uint64_t idx = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= total) return;
  const uint32_t n = 1u << logn;
  const uint64_t row = idx >> logn;
  const uint32_t k = (uint32_t)(idx & (n - 1));
  const uint32_t bk = __brev(k) >> (32 - logn);
  const uint32_t e = (uint32_t)(((uint64_t)(2 * bk + 1) * g) & (2 * n - 1));
  const uint32_t p = __brev((e - 1) >> 1) >> (32 - logn);
  out[idx] = in[(row << logn) + p];
}

// Rescale by the last prime q_k of the input range (FHElium "Eager, Compile, and native
// execution", section "CUDA execution": nearest and truncating rescale).  With X the
// CRT value of a column and x_k = X mod q_k,
//   floor(X / q_k) = (X - x_k) / q_k  ==  (x_l - x_k) * q_k^-1   (mod q_l);
// nearest adds h = floor(q_k / 2) to X first: x_k <- (x_k + h) mod q_k, x_l <- x_l + h.
// x_k is not reduced modulo q_l: y = x_l + (h mod q_l) + M - x_k with M a multiple of
// q_l that is >= q_k stays non-negative and below 2^64, and one Shoup product by
// q_k^-1 (valid for any 64-bit y) gives the quotient residue.
// grid.x: tiles of coefficient pairs; grid.y: batch; grid.z: groups of output limbs.
__global__ __launch_bounds__(kThreads) void rescale_kernel(uint64_t* __restrict__ out,
                                                           const uint64_t* __restrict__ in,
                                                           const ModInfo* __restrict__ mods,
                                                           const RescaleC* __restrict__ tri, uint32_t logn,
                                                           uint32_t limb_begin, uint32_t num_limbs,
                                                           uint32_t nearest) {
  const uint32_t p = blockIdx.x * kThreads + threadIdx.x;
  const uint32_t n = 1u << logn;
  if (2 * p >= n) return;
  const uint32_t outl = num_limbs - 1, k = limb_begin + outl;
  const uint64_t* x = in + (uint64_t)blockIdx.y * num_limbs * n + 2 * p;
  uint64_t* o = out + (uint64_t)blockIdx.y * outl * n + 2 * p;
  const uint64_t qk = mods[k].q;
  const u64x2 xv = ld_stream(x + (uint64_t)outl * n);
  uint64_t xk0 = xv.x, xk1 = xv.y;
  if (nearest) {
    const uint64_t h = qk >> 1;
    xk0 = csub(xk0 + h, qk);
    xk1 = csub(xk1 + h, qk);
  }
  const RescaleC* row = tri + rescale_index(k, limb_begin);
  const uint32_t per = (outl + gridDim.z - 1) / gridDim.z;
  const uint32_t l0 = blockIdx.z * per, l1 = min(outl, l0 + per);
#pragma unroll 4
  for (uint32_t l = l0; l < l1; ++l) {
    const RescaleC c = row[l];
    const uint64_t q = mods[limb_begin + l].q;
    const uint64_t add = c.m + (nearest ? c.half : 0);
    const u64x2 xl = ld_stream(x + (uint64_t)l * n);
    const Wide::Tw w{c.inv, c.inv_shoup};
    u64x2 r;
    r.x = csub(Wide::mul(xl.x + add - xk0, w, q), q);
    r.y = csub(Wide::mul(xl.y + add - xk1, w, q), q);
    st_stream(o + (uint64_t)l * n, r);
  }
}

// Debug input check: how many residues are >= their prime.  One count per block
// (__syncthreads_count), added by one lane through a vector atomic.
__global__ __launch_bounds__(kThreads) void count_noncanonical_kernel(const uint64_t* __restrict__ data,
                                                                      const ModInfo* __restrict__ mods,
                                                                      uint32_t logn, uint32_t num_limbs,
                                                                      uint32_t limb_begin, uint64_t total,
                                                                      unsigned long long* __restrict__ count) {
  const uint64_t idx = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
  int bad = 0;
  if (idx < total) bad = data[idx] >= mods[limb_begin + (uint32_t)((idx >> logn) % num_limbs)].q;
  const int c = __syncthreads_count(bad);
  if (threadIdx.x == 0 && c) atomicAdd(count, (unsigned long long)c);
}

__global__ void zero_counter_kernel(unsigned long long* count) { *count = 0; }

uint32_t blocks_for(uint64_t work) { return (uint32_t)((work + kThreads - 1) / kThreads); }

// launch(first, count) over items [0, items) in parts that keep each launch within
// the launch cap, given the threads one item needs.
template <class F>
hipError_t in_parts(uint64_t items, uint64_t threads_per_item, F&& launch) {
  const uint64_t per = items_per_launch(threads_per_item);
  if (per == 0) return hipErrorNotSupported;
  for (uint64_t i0 = 0; i0 < items; i0 += per) {
    launch(i0, std::min(per, items - i0));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_pointwise(const ntt_plan* p, uint64_t* out, const uint64_t* a, const uint64_t* b, uint64_t batch,
                            uint32_t limb_begin, uint32_t num_limbs, hipStream_t s) {
  const uint64_t poly = (uint64_t)num_limbs * p->n;  // elements per polynomial
  return in_parts(batch, poly / 2, [&](uint64_t b0, uint64_t nb) {
    const uint64_t off = b0 * poly, pairs = nb * poly / 2;
    hipLaunchKernelGGL(pointwise_kernel, dim3(blocks_for(pairs)), dim3(kThreads), 0, s, out + off, a + off, b + off,
                       p->d_mods, p->logn, num_limbs, limb_begin, pairs);
  });
}

hipError_t launch_tensor(const ntt_plan* p, uint64_t* out, const uint64_t* a, const uint64_t* b, uint64_t batch,
                         uint32_t limb_begin, uint32_t num_limbs, hipStream_t s) {
  const uint64_t plane = (uint64_t)num_limbs * p->n;  // elements per component
  return in_parts(batch, plane / 2, [&](uint64_t b0, uint64_t nb) {
    const uint64_t pairs = nb * plane / 2;
    hipLaunchKernelGGL(tensor_kernel, dim3(blocks_for(pairs)), dim3(kThreads), 0, s, out + b0 * 3 * plane,
                       a + b0 * 2 * plane, b + b0 * 2 * plane, p->d_mods, p->logn, num_limbs, limb_begin, pairs);
  });
}

hipError_t launch_automorph(const ntt_plan* p, uint64_t* out, const uint64_t* in, uint64_t g, int domain,
                            uint64_t batch, uint32_t limb_begin, uint32_t num_limbs, hipStream_t s) {
  const uint64_t poly = (uint64_t)num_limbs * p->n;  // elements per polynomial
  if (batch * poly == 0) return hipSuccess;
  const uint32_t two_n = 2 * p->n;
  if (domain != 0)
    return in_parts(batch, poly, [&](uint64_t b0, uint64_t nb) {
      hipLaunchKernelGGL(automorph_ntt_kernel, dim3(blocks_for(nb * poly)), dim3(kThreads), 0, s, out + b0 * poly,
                         in + b0 * poly, p->logn, (uint32_t)(g % two_n), nb * poly);
    });
  const uint32_t h = (uint32_t)host_invmod(g % two_n, two_n);
  // Outputs per thread of the per-element forms (MI355X: 2 beats 1 by 12% and 4 by 5%)
  // and pairs per thread of the pair form (2^16 x 384 rows: one pair 97 us, two 102,
  // four 106; per-element form 114).  Rings whose half is a multiple of a pair block
  // (n >= 512) take the pair form.
  constexpr uint32_t kPer = 2;
  constexpr uint32_t kPairs = 1;
  constexpr uint32_t kPairBlock = kPairs * kThreads;  // even outputs per block
  const uint32_t half = p->n / 2, bpr = half / kPairBlock;
  if (bpr > 0 && half % kPairBlock == 0)
    return in_parts(batch, (uint64_t)num_limbs * bpr * kThreads, [&](uint64_t b0, uint64_t nb) {
      hipLaunchKernelGGL(automorph_coeff_pair_kernel<kPairs>, dim3((uint32_t)(nb * num_limbs * bpr)),
                         dim3(kThreads), 0, s, out + b0 * poly, in + b0 * poly, p->d_mods, p->logn,
                         (uint32_t)(g % two_n), h, num_limbs, limb_begin, bpr);
    });
  return in_parts(batch, poly, [&](uint64_t b0, uint64_t nb) {
    const uint64_t total = nb * poly;
    if (total % (kPer * kThreads) == 0)
      hipLaunchKernelGGL(automorph_coeff_multi_kernel<kPer>, dim3(blocks_for(total / kPer)), dim3(kThreads), 0, s,
                         out + b0 * poly, in + b0 * poly, p->d_mods, p->logn, h, num_limbs, limb_begin, total / kPer);
    else
      hipLaunchKernelGGL(automorph_coeff_kernel, dim3(blocks_for(total)), dim3(kThreads), 0, s, out + b0 * poly,
                         in + b0 * poly, p->d_mods, p->logn, h, num_limbs, limb_begin, total);
  });
}

hipError_t launch_count_noncanonical(const ntt_plan* p, const uint64_t* data, uint64_t rows, uint32_t limb_begin,
                                     uint32_t num_limbs, unsigned long long* count, hipStream_t s) {
  const uint64_t poly = (uint64_t)num_limbs * p->n;
  return in_parts(rows, poly, [&](uint64_t r0, uint64_t nr) {
    hipLaunchKernelGGL(count_noncanonical_kernel, dim3(blocks_for(nr * poly)), dim3(kThreads), 0, s,
                       data + r0 * poly, p->d_mods, p->logn, num_limbs, limb_begin, nr * poly, count);
  });
}

hipError_t launch_zero_counter(unsigned long long* count, hipStream_t s) {
  hipLaunchKernelGGL(zero_counter_kernel, dim3(1), dim3(1), 0, s, count);
  return hipGetLastError();
}

hipError_t launch_rescale(const ntt_plan* p, uint64_t* out, const uint64_t* in, uint64_t batch, uint32_t limb_begin,
                          uint32_t num_limbs, bool nearest, hipStream_t s) {
  if (!batch) return hipSuccess;
  const uint32_t tiles = (p->n / 2 + kThreads - 1) / kThreads;
  // Enough blocks to fill the chip: split the output limbs into groups when the
  // batch is small (each group re-reads the dropped limb, one row of n words).
  constexpr uint64_t kRescaleBlocks = 2048;
  const uint64_t base = (uint64_t)tiles * batch;
  const uint32_t want = (uint32_t)std::min<uint64_t>(num_limbs - 1, (kRescaleBlocks + base - 1) / base);
  const uint32_t groups = std::max(1u, want);
  for (uint64_t b0 = 0; b0 < batch; b0 += 65535) {
    const uint64_t nb = std::min<uint64_t>(65535, batch - b0);
    hipLaunchKernelGGL(rescale_kernel, dim3(tiles, (uint32_t)nb, groups), dim3(kThreads), 0, s,
                       out + b0 * (num_limbs - 1) * p->n, in + b0 * num_limbs * p->n, p->d_mods, p->d_rescale,
                       p->logn, limb_begin, num_limbs, nearest ? 1u : 0u);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace nntt
