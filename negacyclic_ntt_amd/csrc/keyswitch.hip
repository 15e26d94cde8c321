// Rotation key-switch (placeholder until the kernels land).
#include "internal.h"

struct ntt_ks_plan {
  int unused;
};

extern "C" int keyswitch_plan_create(ntt_ks_plan** out, const ntt_plan*, uint32_t, uint32_t, uint32_t) {
  if (out) *out = nullptr;
  return NTT_EUNSUPPORTED;
}
extern "C" int keyswitch_workspace_size(const ntt_ks_plan*, uint64_t, size_t*) { return NTT_EUNSUPPORTED; }
extern "C" int keyswitch(const ntt_ks_plan*, uint64_t*, const uint64_t*, const uint64_t*, uint64_t, uint64_t, void*,
                         size_t, void*) {
  return NTT_EUNSUPPORTED;
}
extern "C" void keyswitch_plan_destroy(ntt_ks_plan*) {}
