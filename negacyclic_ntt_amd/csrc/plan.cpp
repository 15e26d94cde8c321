// Host side of the transform plan: argument validation, prime search, the
// primitive root psi, bit-reversed twiddle tables with Shoup companions, and the
// upload to the device.
//
// Readings (the pages fix none of these; each is the plain choice):
//   - psi is the smallest x >= 2 with x^n == -1 (mod q) unless the caller
//     passes one; any primitive 2n-th root gives a valid transform, so the only
//     requirement is that every user of a plan agrees on it.
//   - NTT-domain order is bit-reversed: the table psi^brv(k) drives an in-place
//     decimation-in-time transform that needs no reordering pass.
#include <string.h>

#include <algorithm>
#include <new>
#include <vector>

#include "internal.h"

namespace nntt {

using u128 = unsigned __int128;

uint64_t host_mulmod(uint64_t a, uint64_t b, uint64_t q) { return (uint64_t)(((u128)a * b) % q); }

uint64_t host_powmod(uint64_t b, uint64_t e, uint64_t q) {
  uint64_t r = 1 % q;
  b %= q;
  for (; e; e >>= 1) {
    if (e & 1) r = host_mulmod(r, b, q);
    b = host_mulmod(b, b, q);
  }
  return r;
}

// Extended Euclid (q need not be prime for this helper; gcd(a, q) must be 1).
uint64_t host_invmod(uint64_t a, uint64_t q) {
  __int128 t = 0, nt = 1, r = q, nr = a % q;
  while (nr) {
    __int128 quo = r / nr, tmp;
    tmp = t - quo * nt;
    t = nt;
    nt = tmp;
    tmp = r - quo * nr;
    r = nr;
    nr = tmp;
  }
  if (t < 0) t += q;
  return (uint64_t)t;
}

// Deterministic Miller-Rabin for 64-bit n with the seven bases found by J. Sinclair
// (2, 325, 9375, 28178, 450775, 9780504, 1795265022).
bool host_is_prime(uint64_t n) {
  if (n < 2) return false;
  static const uint64_t small[] = {2, 3, 5, 7, 11, 13, 17, 19, 23, 29, 31, 37};
  for (uint64_t p : small) {
    if (n == p) return true;
    if (n % p == 0) return false;
  }
  uint64_t d = n - 1;
  int s = 0;
  while (!(d & 1)) d >>= 1, ++s;
  static const uint64_t bases[] = {2, 325, 9375, 28178, 450775, 9780504, 1795265022};
  for (uint64_t a0 : bases) {
    uint64_t a = a0 % n;
    if (a == 0) continue;
    uint64_t x = host_powmod(a, d, n);
    if (x == 1 || x == n - 1) continue;
    bool composite = true;
    for (int r = 1; r < s && composite; ++r) {
      x = host_mulmod(x, x, n);
      if (x == n - 1) composite = false;
    }
    if (composite) return false;
  }
  return true;
}

Barrett host_barrett(uint64_t q) {
  Barrett b;
  b.q = q;
  b.k = 64 - __builtin_clzll(q);
  b.mu = (uint64_t)(((u128)1 << (2 * b.k)) / q);
  return b;
}

// The row-pass layout of the two-pass split (internal.h, row_tw_permuted) for one
// prime's table t[0, 2^logn): within each stage block s >= log N1 + 4 and each row r,
// entry (u, j) moves from u 2^v + j to j 2^4 + u (v = s - log N1 - 4).
template <class Tw>
static void permute_row_stages(Tw* t, uint32_t logn) {
  const uint32_t logn1 = logn - kPermRowLog, n1 = 1u << logn1, g = 1u << kPermRowS0;
  std::vector<Tw> tmp;
  for (uint32_t s = logn1 + kPermRowS0; s < logn; ++s) {
    const uint32_t v = s - logn1 - kPermRowS0, span = g << v;
    for (uint32_t r = 0; r < n1; ++r) {
      Tw* blk = t + (1u << s) + (size_t)r * span;
      tmp.assign(blk, blk + span);
      for (uint32_t u = 0; u < g; ++u)
        for (uint32_t j = 0; j < (1u << v); ++j) blk[j * g + u] = tmp[(u << v) + j];
    }
  }
}

static unsigned bitrev(unsigned x, unsigned bits) {
  unsigned r = 0;
  for (unsigned i = 0; i < bits; ++i) r = (r << 1) | ((x >> i) & 1u);
  return r;
}

// An element of order exactly 2n, then the smallest of its odd powers (the set of
// all x with x^n == -1).
static uint64_t smallest_psi(uint64_t q, uint64_t n) {
  uint64_t e = (q - 1) / (2 * n), r = 0;
  for (uint64_t x = 2; x < q && !r; ++x) {
    uint64_t c = host_powmod(x, e, q);
    if (host_powmod(c, n, q) == q - 1) r = c;
  }
  if (!r) return 0;
  uint64_t best = r, step = host_mulmod(r, r, q), cur = r;
  for (uint64_t k = 1; k < n; ++k) {
    cur = host_mulmod(cur, step, q);
    best = std::min(best, cur);
  }
  return best;
}

DeviceGuard::DeviceGuard(int dev) {
  if (hipGetDevice(&prev) != hipSuccess) return;
  ok = prev == dev || hipSetDevice(dev) == hipSuccess;
}
DeviceGuard::~DeviceGuard() {
  int cur = -1;
  if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
}

}  // namespace nntt

using namespace nntt;

extern "C" const char* ntt_status_string(int s) {
  switch (s) {
    case NTT_OK: return "ok";
    case NTT_EINVAL: return "invalid argument";
    case NTT_EUNSUPPORTED: return "unsupported";
    case NTT_ENOMEM: return "out of memory";
    case NTT_EDEVICE: return "device error";
    case NTT_EOVERLAP: return "forbidden overlap";
    default: return "unknown status";
  }
}

extern "C" int ntt_find_primes(uint32_t bits, uint32_t n, uint32_t count, uint64_t* out) {
  if (bits < 3 || bits > 62 || n < 2 || n > (1u << kMaxLogN) || (n & (n - 1)) || (count && !out)) return NTT_EINVAL;
  uint64_t two_n = 2ull * n;
  uint64_t c = (((1ull << bits) - 2) / two_n) * two_n + 1;
  uint32_t got = 0;
  for (; got < count && c > two_n; c -= two_n)
    if (host_is_prime(c)) out[got++] = c;
  return got == count ? NTT_OK : NTT_EINVAL;
}

static void free_device(ntt_plan* p) {
  if (p->device < 0) return;
  DeviceGuard g(p->device);
  (void)hipFree(p->d_fwd);
  (void)hipFree(p->d_inv);
  (void)hipFree(p->d_fwd60);
  (void)hipFree(p->d_inv60);
  (void)hipFree(p->d_fwd32);
  (void)hipFree(p->d_inv32);
  (void)hipFree(p->d_mods);
  (void)hipFree(p->d_rescale);
  (void)hipFree(p->d_check);
  p->d_fwd = p->d_inv = nullptr;
  p->d_fwd60 = p->d_inv60 = nullptr;
  p->d_fwd32 = p->d_inv32 = nullptr;
  p->d_mods = nullptr;
  p->d_rescale = nullptr;
  p->d_check = nullptr;
}

// Rescale constants for every pair l < k.  The inverses of q_k mod q_l for all k > l
// share one modular inversion per l (Montgomery's simultaneous inversion: invert the
// running product once, then peel the factors off from the back).
static int rescale_triangle(const uint64_t* primes, uint32_t L, std::vector<RescaleC>* out) {
  try {
    out->assign(rescale_index(L, 0), RescaleC{0, 0, 0, 0});
  } catch (const std::bad_alloc&) {
    return NTT_ENOMEM;
  }
  std::vector<uint64_t> pre(L + 1);
  for (uint32_t l = 0; l + 1 < L; ++l) {
    const uint64_t ql = primes[l];
    pre[l + 1] = 1;  // pre[k + 1] = prod_{l < j <= k} (q_j mod q_l)
    for (uint32_t k = l + 1; k < L; ++k) pre[k + 1] = host_mulmod(pre[k], primes[k] % ql, ql);
    uint64_t inv_run = host_invmod(pre[L], ql);  // (prod_{l < j < L} q_j)^-1
    for (uint32_t k = L - 1; k > l; --k) {
      const uint64_t inv = host_mulmod(inv_run, pre[k], ql);  // q_k^-1
      inv_run = host_mulmod(inv_run, primes[k] % ql, ql);
      RescaleC& c = (*out)[rescale_index(k, l)];
      c.inv = inv;
      c.inv_shoup = (uint64_t)(((u128)inv << 64) / ql);
      c.m = ql * ((primes[k] + ql - 1) / ql);
      c.half = (primes[k] / 2) % ql;
    }
  }
  return NTT_OK;
}

template <class T>
static int upload(T** dst, const void* src, size_t bytes) {
  if (hipMalloc((void**)dst, bytes) != hipSuccess) {
    *dst = nullptr;
    return NTT_ENOMEM;
  }
  if (hipMemcpy(*dst, src, bytes, hipMemcpyHostToDevice) != hipSuccess) return NTT_EDEVICE;
  return NTT_OK;
}

extern "C" int ntt_plan_create(ntt_plan** out, uint32_t n, const uint64_t* primes, uint32_t num_primes,
                               const uint64_t* psi, int device) {
  if (!out) return NTT_EINVAL;
  *out = nullptr;
  if (n < 2 || n > (1u << kMaxLogN) || (n & (n - 1))) return NTT_EINVAL;
  if (!primes || num_primes == 0 || num_primes > kMaxPrimes) return NTT_EINVAL;
  if (device < -1) return NTT_EINVAL;
  if (device >= 0) {
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || device >= count) return NTT_EDEVICE;
  }
  uint64_t two_n = 2ull * n;
  for (uint32_t i = 0; i < num_primes; ++i) {
    uint64_t q = primes[i];
    if (q < 3 || q >= (1ull << 62) || q % two_n != 1 || !host_is_prime(q)) return NTT_EINVAL;
    for (uint32_t j = 0; j < i; ++j)
      if (primes[j] == q) return NTT_EINVAL;
    if (psi && (psi[i] == 0 || psi[i] >= q || host_powmod(psi[i], n, q) != q - 1)) return NTT_EINVAL;
  }

  ntt_plan* p = new (std::nothrow) ntt_plan;
  if (!p) return NTT_ENOMEM;
  p->n = n;
  p->logn = 31 - __builtin_clz(n);
  p->num_primes = num_primes;
  p->device = device;
  p->primes.assign(primes, primes + num_primes);
  p->psis.resize(num_primes);
  p->narrow.resize(num_primes);
  p->below60.resize(num_primes);
  size_t tn = (size_t)num_primes * n;
  p->h_fwd.resize(tn);
  p->h_fwd_sh.resize(tn);
  p->h_inv.resize(tn);
  p->h_inv_sh.resize(tn);
  p->h_mods.resize(num_primes);
  std::vector<Wide::Tw> fwd(tn), inv(tn);
  std::vector<Wide60::Tw> fwd60(tn, Wide60::Tw{0, 0}), inv60(tn, Wide60::Tw{0, 0});
  std::vector<Narrow::Tw> fwd32(tn, Narrow::Tw{0, 0}), inv32(tn, Narrow::Tw{0, 0});
  std::vector<uint64_t> pw(n), ipw(n);

  for (uint32_t l = 0; l < num_primes; ++l) {
    uint64_t q = primes[l];
    uint64_t ps = psi ? psi[l] : smallest_psi(q, n);
    if (!ps) {
      delete p;
      return NTT_EINVAL;
    }
    uint64_t ips = host_invmod(ps, q);
    p->psis[l] = ps;
    p->narrow[l] = q < (1ull << 30);
    p->below60[l] = q < (1ull << 60);
    pw[0] = ipw[0] = 1;
    for (uint32_t e = 1; e < n; ++e) {
      pw[e] = host_mulmod(pw[e - 1], ps, q);
      ipw[e] = host_mulmod(ipw[e - 1], ips, q);
    }
    for (uint32_t k = 0; k < n; ++k) {
      size_t i = (size_t)l * n + k;
      uint64_t w = pw[bitrev(k, p->logn)], iw = ipw[bitrev(k, p->logn)];
      uint64_t wsh = (uint64_t)(((u128)w << 64) / q), iwsh = (uint64_t)(((u128)iw << 64) / q);
      p->h_fwd[i] = w;
      p->h_fwd_sh[i] = wsh;
      p->h_inv[i] = iw;
      p->h_inv_sh[i] = iwsh;
      fwd[i] = Wide::Tw{w, wsh};
      inv[i] = Wide::Tw{iw, iwsh};
      if (p->below60[l]) {  // floor(w 2^62 / q) = floor(floor(w 2^64 / q) / 4)
        fwd60[i] = Wide60::Tw{w, wsh >> 2};
        inv60[i] = Wide60::Tw{iw, iwsh >> 2};
      }
      if (p->narrow[l]) {
        fwd32[i] = Narrow::Tw{(uint32_t)w, (uint32_t)(((uint64_t)w << 32) / q)};
        inv32[i] = Narrow::Tw{(uint32_t)iw, (uint32_t)(((uint64_t)iw << 32) / q)};
      }
    }
    if (row_tw_permuted(p->logn)) {
      permute_row_stages(fwd.data() + (size_t)l * n, p->logn);
      permute_row_stages(inv.data() + (size_t)l * n, p->logn);
      permute_row_stages(fwd60.data() + (size_t)l * n, p->logn);
      permute_row_stages(inv60.data() + (size_t)l * n, p->logn);
      permute_row_stages(fwd32.data() + (size_t)l * n, p->logn);
      permute_row_stages(inv32.data() + (size_t)l * n, p->logn);
    }
    ModInfo& m = p->h_mods[l];
    memset(&m, 0, sizeof(m));
    m.q = q;
    m.n_inv = host_invmod(n % q, q);
    m.n_inv_shoup = (uint64_t)(((u128)m.n_inv << 64) / q);
    m.n_inv_shoup60 = p->below60[l] ? (uint64_t)(((u128)m.n_inv << 62) / q) : 0;
    if (p->narrow[l]) {
      m.n_inv32 = (uint32_t)m.n_inv;
      m.n_inv_shoup32 = (uint32_t)(((uint64_t)m.n_inv << 32) / q);
    }
    m.w1n = host_mulmod(p->h_inv[(size_t)l * n + 1], m.n_inv, q);
    m.w1n_shoup = (uint64_t)(((u128)m.w1n << 64) / q);
    m.w1n_shoup60 = p->below60[l] ? (uint64_t)(((u128)m.w1n << 62) / q) : 0;
    if (p->narrow[l]) {
      m.w1n32 = (uint32_t)m.w1n;
      m.w1n_shoup32 = (uint32_t)(((uint64_t)m.w1n << 32) / q);
    }
    m.br = host_barrett(q);
    uint64_t inv = q;  // Newton: q * q == 1 mod 8, each step doubles the correct bits
    for (int it = 0; it < 5; ++it) inv *= 2 - q * inv;
    m.mont_ninv = 0 - inv;
    m.r64 = (uint64_t)(((u128)1 << 64) % q);
    m.r64_shoup = (uint64_t)(((u128)m.r64 << 64) / q);
  }

  if (device >= 0) {
    DeviceGuard g(device);
    int rc = g.ok ? NTT_OK : NTT_EDEVICE;
    if (rc == NTT_OK) rc = upload(&p->d_fwd, fwd.data(), tn * sizeof(Wide::Tw));
    if (rc == NTT_OK) rc = upload(&p->d_inv, inv.data(), tn * sizeof(Wide::Tw));
    if (rc == NTT_OK) rc = upload(&p->d_fwd60, fwd60.data(), tn * sizeof(Wide60::Tw));
    if (rc == NTT_OK) rc = upload(&p->d_inv60, inv60.data(), tn * sizeof(Wide60::Tw));
    if (rc == NTT_OK) rc = upload(&p->d_fwd32, fwd32.data(), tn * sizeof(Narrow::Tw));
    if (rc == NTT_OK) rc = upload(&p->d_inv32, inv32.data(), tn * sizeof(Narrow::Tw));
    if (rc == NTT_OK) rc = upload(&p->d_mods, p->h_mods.data(), num_primes * sizeof(ModInfo));
    if (rc == NTT_OK) {
      const unsigned long long zero = 0;
      rc = upload(&p->d_check, &zero, sizeof(zero));
    }
    if (rc == NTT_OK && num_primes > 1) {
      std::vector<RescaleC> tri;
      rc = rescale_triangle(primes, num_primes, &tri);
      if (rc == NTT_OK) rc = upload(&p->d_rescale, tri.data(), tri.size() * sizeof(RescaleC));
    }
    if (rc != NTT_OK) {
      free_device(p);
      delete p;
      return rc;
    }
  }
  *out = p;
  return NTT_OK;
}

extern "C" int ntt_plan_get_tables(const ntt_plan* p, uint32_t limb, uint64_t* psi_out, uint64_t* fwd,
                                   uint64_t* fwd_shoup, uint64_t* inv, uint64_t* inv_shoup) {
  if (!p || limb >= p->num_primes) return NTT_EINVAL;
  size_t off = (size_t)limb * p->n, bytes = p->n * sizeof(uint64_t);
  if (psi_out) *psi_out = p->psis[limb];
  if (fwd) memcpy(fwd, p->h_fwd.data() + off, bytes);
  if (fwd_shoup) memcpy(fwd_shoup, p->h_fwd_sh.data() + off, bytes);
  if (inv) memcpy(inv, p->h_inv.data() + off, bytes);
  if (inv_shoup) memcpy(inv_shoup, p->h_inv_sh.data() + off, bytes);
  return NTT_OK;
}

extern "C" int ntt_plan_info(const ntt_plan* p, uint32_t* n, uint32_t* num_primes, int* device) {
  if (!p) return NTT_EINVAL;
  if (n) *n = p->n;
  if (num_primes) *num_primes = p->num_primes;
  if (device) *device = p->device;
  return NTT_OK;
}

extern "C" int ntt_plan_prime(const ntt_plan* p, uint32_t limb, uint64_t* q) {
  if (!p || !q || limb >= p->num_primes) return NTT_EINVAL;
  *q = p->primes[limb];
  return NTT_OK;
}

extern "C" void ntt_plan_destroy(ntt_plan* p) {
  if (!p) return;
  free_device(p);
  delete p;
}
