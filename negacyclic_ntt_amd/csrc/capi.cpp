// C-ABI entry points: argument validation (before anything is enqueued), device
// selection and dispatch to the launchers.  Follows the FHElium native-call
// conventions ("Eager, Compile, and native execution", sections "Schema
// registration and device dispatch" and "CUDA execution"): shapes, ranges and
// forbidden overlap are checked first; work goes on the caller's stream with no
// host synchronisation; launch failures are reported, asynchronous faults surface
// at the caller's next synchronisation.
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "internal.h"

using namespace nntt;

// ---- debug input checks ------------------------------------------------------------
// Off by default.  NTT_CHECK_INPUTS (any value but "" or "0") turns them on for the
// process; ntt_set_debug_checks overrides it.  Each check uses the plan's one device
// counter and waits on the caller's stream, so checks are serialised process-wide.
namespace {
std::atomic<int> g_debug{-1};
std::mutex g_debug_mu;

bool debug_checks_enabled() {
  int v = g_debug.load();
  if (v < 0) {
    const char* e = getenv("NTT_CHECK_INPUTS");
    v = (e && *e && strcmp(e, "0") != 0) ? 1 : 0;
    int expected = -1;
    g_debug.compare_exchange_strong(expected, v);
    v = g_debug.load();
  }
  return v == 1;
}
}  // namespace

namespace nntt {
int debug_check_inputs(const ntt_plan* p, const uint64_t* data, uint64_t rows, uint32_t limb_begin,
                       uint32_t num_limbs, hipStream_t s) {
  if (!debug_checks_enabled() || rows == 0) return NTT_OK;
  std::lock_guard<std::mutex> lock(g_debug_mu);
  DeviceGuard g(p->device);
  if (!g.ok) return NTT_EDEVICE;
  unsigned long long h = 0;
  if (launch_zero_counter(p->d_check, s) != hipSuccess ||
      launch_count_noncanonical(p, data, rows, limb_begin, num_limbs, p->d_check, s) != hipSuccess ||
      hipMemcpyAsync(&h, p->d_check, sizeof(h), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return NTT_EDEVICE;
  return h ? NTT_EINVAL : NTT_OK;
}
}  // namespace nntt

extern "C" void ntt_set_debug_checks(int on) { g_debug.store(on ? 1 : 0); }

namespace nntt {
namespace {
std::atomic<uint64_t> g_max_threads{kMaxLaunchThreads};
}
uint64_t max_launch_threads() { return g_max_threads.load(std::memory_order_relaxed); }
}  // namespace nntt

extern "C" int ntt_set_max_launch_threads(uint64_t threads) {
  if (threads != 0 && threads < 256) return NTT_EINVAL;
  nntt::g_max_threads.store(threads == 0 ? nntt::kMaxLaunchThreads : std::min(threads, nntt::kMaxLaunchThreads));
  return NTT_OK;
}

namespace {

constexpr uint64_t kMaxElements = 1ull << 36;  // 512 GiB of residues: beyond any device

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Half-open byte ranges [a, a + na) and [b, b + nb).
bool overlaps(const void* a, uint64_t na, const void* b, uint64_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return na && nb && x < y + nb && y < x + na;
}

// out may equal `in` exactly (if allowed) but may not overlap it otherwise.
bool bad_overlap(const void* out, const void* in, uint64_t bytes, bool exact_ok) {
  if (out == in) return !exact_ok && bytes != 0;
  return overlaps(out, bytes, in, bytes);
}

int check_plan_range(const ntt_plan* p, uint64_t batch, uint32_t limb_begin, uint32_t num_limbs,
                     uint64_t components, uint64_t* elements) {
  if (!p) return NTT_EINVAL;
  if (p->device < 0) return NTT_EDEVICE;
  if (num_limbs == 0 || limb_begin >= p->num_primes || num_limbs > p->num_primes - limb_begin) return NTT_EINVAL;
  const uint64_t per = (uint64_t)num_limbs * p->n * components;
  if (batch > kMaxElements / per) return NTT_EUNSUPPORTED;
  *elements = batch * per;
  return NTT_OK;
}

// hipErrorNotSupported: a launcher's own refusal (one polynomial beyond the launch cap).
int status_of(hipError_t e) {
  return e == hipSuccess ? NTT_OK : e == hipErrorNotSupported ? NTT_EUNSUPPORTED : NTT_EDEVICE;
}

int transform(const ntt_plan* p, uint64_t* data, uint64_t batch, uint32_t limb_begin, uint32_t num_limbs,
              void* stream, bool inverse) {
  uint64_t elems = 0;
  int rc = check_plan_range(p, batch, limb_begin, num_limbs, 1, &elems);
  if (rc) return rc;
  if (!elems) return NTT_OK;
  if (!data || !aligned16(data)) return NTT_EINVAL;
  if ((rc = debug_check_inputs(p, data, batch, limb_begin, num_limbs, (hipStream_t)stream))) return rc;
  DeviceGuard g(p->device);
  if (!g.ok) return NTT_EDEVICE;
  return status_of(launch_ntt(p, data, batch, limb_begin, num_limbs, inverse, (hipStream_t)stream));
}

bool valid_galois(const ntt_plan* p, uint64_t g) { return (g & 1) && g < 2ull * p->n; }

}  // namespace

extern "C" int ntt_forward(const ntt_plan* p, uint64_t* data, uint64_t batch, uint32_t limb_begin,
                           uint32_t num_limbs, void* stream) {
  return transform(p, data, batch, limb_begin, num_limbs, stream, false);
}

extern "C" int ntt_inverse(const ntt_plan* p, uint64_t* data, uint64_t batch, uint32_t limb_begin,
                           uint32_t num_limbs, void* stream) {
  return transform(p, data, batch, limb_begin, num_limbs, stream, true);
}

extern "C" int ntt_forward_galois(const ntt_plan* p, uint64_t* out, const uint64_t* in, uint64_t galois_elt,
                                  uint64_t batch, uint32_t limb_begin, uint32_t num_limbs, void* stream) {
  uint64_t elems = 0;
  int rc = check_plan_range(p, batch, limb_begin, num_limbs, 1, &elems);
  if (rc) return rc;
  if (!valid_galois(p, galois_elt)) return NTT_EINVAL;
  if (!elems) return NTT_OK;
  if (!out || !in || !aligned16(out) || !aligned16(in)) return NTT_EINVAL;
  if (bad_overlap(out, in, elems * 8, true)) return NTT_EOVERLAP;
  if ((rc = debug_check_inputs(p, in, batch, limb_begin, num_limbs, (hipStream_t)stream))) return rc;
  DeviceGuard g(p->device);
  if (!g.ok) return NTT_EDEVICE;
  return status_of(launch_ntt_galois(p, out, in, galois_elt, batch, limb_begin, num_limbs, (hipStream_t)stream));
}

extern "C" int poly_mul_ntt(const ntt_plan* p, uint64_t* out, const uint64_t* a, const uint64_t* b, uint64_t batch,
                            uint32_t limb_begin, uint32_t num_limbs, void* stream) {
  uint64_t elems = 0;
  int rc = check_plan_range(p, batch, limb_begin, num_limbs, 1, &elems);
  if (rc) return rc;
  if (!elems) return NTT_OK;
  if (!out || !a || !b || !aligned16(out) || !aligned16(a) || !aligned16(b)) return NTT_EINVAL;
  if (bad_overlap(out, a, elems * 8, true) || bad_overlap(out, b, elems * 8, true)) return NTT_EOVERLAP;
  if ((rc = debug_check_inputs(p, a, batch, limb_begin, num_limbs, (hipStream_t)stream))) return rc;
  if ((rc = debug_check_inputs(p, b, batch, limb_begin, num_limbs, (hipStream_t)stream))) return rc;
  DeviceGuard g(p->device);
  if (!g.ok) return NTT_EDEVICE;
  return status_of(launch_pointwise(p, out, a, b, batch, limb_begin, num_limbs, (hipStream_t)stream));
}

extern "C" int ct_tensor_ntt(const ntt_plan* p, uint64_t* out, const uint64_t* a, const uint64_t* b, uint64_t batch,
                             uint32_t limb_begin, uint32_t num_limbs, void* stream) {
  uint64_t elems = 0;
  int rc = check_plan_range(p, batch, limb_begin, num_limbs, 3, &elems);
  if (rc) return rc;
  if (!elems) return NTT_OK;
  if (!out || !a || !b || !aligned16(out) || !aligned16(a) || !aligned16(b)) return NTT_EINVAL;
  const uint64_t in_bytes = elems / 3 * 2 * 8, out_bytes = elems * 8;
  if (overlaps(out, out_bytes, a, in_bytes) || overlaps(out, out_bytes, b, in_bytes)) return NTT_EOVERLAP;
  if ((rc = debug_check_inputs(p, a, 2 * batch, limb_begin, num_limbs, (hipStream_t)stream))) return rc;
  if ((rc = debug_check_inputs(p, b, 2 * batch, limb_begin, num_limbs, (hipStream_t)stream))) return rc;
  DeviceGuard g(p->device);
  if (!g.ok) return NTT_EDEVICE;
  return status_of(launch_tensor(p, out, a, b, batch, limb_begin, num_limbs, (hipStream_t)stream));
}

extern "C" int ct_tensor_coeff(const ntt_plan* p, uint64_t* out, const uint64_t* a, const uint64_t* b,
                               uint64_t batch, uint32_t limb_begin, uint32_t num_limbs, void* stream) {
  uint64_t elems = 0;
  int rc = check_plan_range(p, batch, limb_begin, num_limbs, 3, &elems);
  if (rc) return rc;
  if (!chain_supported(p)) return NTT_EUNSUPPORTED;
  if (!elems) return NTT_OK;
  if (!out || !a || !b || !aligned16(out) || !aligned16(a) || !aligned16(b)) return NTT_EINVAL;
  const uint64_t in_bytes = elems / 3 * 2 * 8, out_bytes = elems * 8;
  if (overlaps(out, out_bytes, a, in_bytes) || overlaps(out, out_bytes, b, in_bytes)) return NTT_EOVERLAP;
  if ((rc = debug_check_inputs(p, a, 2 * batch, limb_begin, num_limbs, (hipStream_t)stream))) return rc;
  if ((rc = debug_check_inputs(p, b, 2 * batch, limb_begin, num_limbs, (hipStream_t)stream))) return rc;
  DeviceGuard g(p->device);
  if (!g.ok) return NTT_EDEVICE;
  return status_of(launch_ct_tensor_coeff(p, out, a, b, batch, limb_begin, num_limbs, (hipStream_t)stream));
}

extern "C" int automorph(const ntt_plan* p, uint64_t* out, const uint64_t* in, uint64_t galois_elt, int domain,
                         uint64_t batch, uint32_t limb_begin, uint32_t num_limbs, void* stream) {
  uint64_t elems = 0;
  int rc = check_plan_range(p, batch, limb_begin, num_limbs, 1, &elems);
  if (rc) return rc;
  if (!valid_galois(p, galois_elt) || (domain != 0 && domain != 1)) return NTT_EINVAL;
  if (!elems) return NTT_OK;
  if (!out || !in || !aligned16(out) || !aligned16(in)) return NTT_EINVAL;
  if (overlaps(out, elems * 8, in, elems * 8)) return NTT_EOVERLAP;
  if ((rc = debug_check_inputs(p, in, batch, limb_begin, num_limbs, (hipStream_t)stream))) return rc;
  DeviceGuard g(p->device);
  if (!g.ok) return NTT_EDEVICE;
  return status_of(launch_automorph(p, out, in, galois_elt, domain, batch, limb_begin, num_limbs,
                                    (hipStream_t)stream));
}

extern "C" int rescale(const ntt_plan* p, uint64_t* out, const uint64_t* in, int mode, uint64_t batch,
                       uint32_t limb_begin, uint32_t num_limbs, void* stream) {
  uint64_t elems = 0;
  int rc = check_plan_range(p, batch, limb_begin, num_limbs, 1, &elems);
  if (rc) return rc;
  if (num_limbs < 2 || (mode != 0 && mode != 1)) return NTT_EINVAL;
  if (!elems) return NTT_OK;
  if (!out || !in || !aligned16(out) || !aligned16(in)) return NTT_EINVAL;
  const uint64_t out_elems = elems / num_limbs * (num_limbs - 1);
  if (overlaps(out, out_elems * 8, in, elems * 8)) return NTT_EOVERLAP;
  if ((rc = debug_check_inputs(p, in, batch, limb_begin, num_limbs, (hipStream_t)stream))) return rc;
  DeviceGuard g(p->device);
  if (!g.ok) return NTT_EDEVICE;
  return status_of(launch_rescale(p, out, in, batch, limb_begin, num_limbs, mode == 1, (hipStream_t)stream));
}

extern "C" int ntt_count_noncanonical(const ntt_plan* p, const uint64_t* data, uint64_t batch, uint32_t limb_begin,
                                      uint32_t num_limbs, uint64_t* count, void* stream) {
  uint64_t elems = 0;
  int rc = check_plan_range(p, batch, limb_begin, num_limbs, 1, &elems);
  if (rc) return rc;
  if (!count || ((uintptr_t)count & 7u)) return NTT_EINVAL;
  if (!elems) return NTT_OK;
  if (!data || !aligned16(data)) return NTT_EINVAL;
  if (overlaps(count, 8, data, elems * 8)) return NTT_EOVERLAP;
  DeviceGuard g(p->device);
  if (!g.ok) return NTT_EDEVICE;
  return status_of(launch_count_noncanonical(p, data, batch, limb_begin, num_limbs, (unsigned long long*)count,
                                             (hipStream_t)stream));
}
