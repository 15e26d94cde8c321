// Allocation-free rotation key-switch: keyswitch() with its workspace in a static
// device array instead of a caller-supplied buffer, for callers that cannot allocate
// device memory on the call path (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// The array lives in this translation unit's code object, so a GPU holds it once the
// object is loaded there (at the first call on that device) until the process ends.
// In host code `scratch` names a host-side stand-in, not device memory: its device
// address on each GPU comes from hipGetSymbolAddress, taken once per device with that
// device current, and only that address is ever passed to a kernel.
#include <mutex>

#include "internal.h"

namespace {

// One key-switch of one ciphertext at n = 2^16 over Q u P = 32 primes with 3 digits:
// (dnum + 2) (Q + P) n 8 bytes = 5 x 32 x 65536 x 8 = 80 MiB.
constexpr size_t kScratchBytes = 80ull << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of `scratch` on device `dev` (looked up once per device).
int scratch_on(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return NTT_EDEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    nntt::DeviceGuard g(dev);
    if (!g.ok) return NTT_EDEVICE;
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return NTT_EDEVICE;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return NTT_OK;
}

}  // namespace

extern "C" int keyswitch_noalloc(const ntt_ks_plan* plan, uint64_t* out, const uint64_t* ct, const uint64_t* ksk,
                                 uint64_t galois_elt, uint64_t batch, void* stream) {
  if (!plan) return NTT_EINVAL;
  size_t need = 0;
  const int rc = keyswitch_workspace_size(plan, batch, &need);
  if (rc != NTT_OK) return rc;
  if (need > kScratchBytes) return NTT_EUNSUPPORTED;  // beyond the static workspace: nothing launched
  if (batch == 0) return keyswitch(plan, out, ct, ksk, galois_elt, 0, nullptr, 0, stream);
  void* ws = nullptr;
  const int dr = scratch_on(nntt::ks_plan_device(plan), &ws);
  if (dr != NTT_OK) return dr;
  // Every byte of the workspace that a key-switch reads it has written first in the
  // same call (ModUp fills the extended digits, the key product the accumulators), so
  // nothing needs clearing between calls.
  return keyswitch(plan, out, ct, ksk, galois_elt, batch, ws, kScratchBytes, stream);
}
