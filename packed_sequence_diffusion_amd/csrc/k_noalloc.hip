// dit_adaln_eval_noalloc: dit_adaln_eval without its scratch argument, for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation).  The Z-Image
// timestep MLP's scratch (its hidden vector and the sinusoid / timestep
// embedding slot, temb_hidden + temb_freq floats) lives in a file-scope
// device array of DIT_NOALLOC_TEMB_MAX floats, one copy per GPU for the life
// of the process.  Every call on a GPU uses that GPU's copy: calls that
// overlap on one GPU (different streams, or host threads) race on it.
// Nothing in it needs to start at zero: each call writes every element it
// reads before reading it.
#include <mutex>

#include "../../include/dit.h"
#include "api_internal.h"

using namespace dit_host;

namespace {

static __device__ __align__(256) float scratch[DIT_NOALLOC_TEMB_MAX];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`.  In host code the
// array's name only stands in for the symbol: kernels get this address.
dit_status scratch_ptr(float** out) {
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(DIT_EUNSUPPORTED, "device %d beyond the %d the scratch table holds", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (!p) return fail(DIT_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = (float*)p;
  }
  *out = g_scratch_ptr[dev];
  return DIT_OK;
}

}  // namespace

extern "C" dit_status dit_adaln_eval_noalloc(const dit_config* c, const void* prepared,
                                             const double* sigmas, int32_t n_sigmas,
                                             float* mods_out, void* stream) {
  DIT_TRY(check_config(c));
  if (!has_mods(c)) return fail(DIT_EUNSUPPORTED, "variant %d has no modulation", c->variant);
  if (!prepared || !mods_out) return fail(DIT_EINVAL, "prepared/mods_out is NULL");
  DIT_TRY(check_sigmas(c, sigmas, n_sigmas));
  float* temb = nullptr;
  if (temb_variant(c)) {
    const long long need = (long long)c->temb_hidden + (long long)c->temb_freq;
    if (need > DIT_NOALLOC_TEMB_MAX)
      return fail(DIT_EUNSUPPORTED,
                  "the timestep MLP needs %lld floats of scratch; dit_adaln_eval_noalloc holds %d",
                  need, DIT_NOALLOC_TEMB_MAX);
    DIT_TRY(scratch_ptr(&temb));
  }
  return launch_mods(c, prepared, sigmas, mods_out, temb, (hipStream_t)stream);
}
