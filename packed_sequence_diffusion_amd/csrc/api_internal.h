// Host-side helpers shared by the C-ABI translation units (dit_api.cpp: configs,
// layouts, weight preparation and the block; dit_model.cpp: evaluation layouts,
// slot plans and the whole-model forwards).  Not part of the public ABI.
#pragma once
#include <new>
#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "../../include/dit.h"

namespace dit_host {

constexpr int kMaxSlots = 8;  // timestep slots of one block, at most
// Tokens of one call, at most: every int product the kernels form from a row
// count (rows x head-dim pairs of the cos/sin table, grid sizes) stays below 2^31.
constexpr int kMaxTokens = 1 << 24;
inline bool bad_tokens(long long n) { return n < 0 || n > kMaxTokens; }

constexpr size_t kNone = SIZE_MAX;  // offset of a buffer a variant does not have
constexpr size_t kAlign = 256;      // alignment of every workspace / prepared-weight region

inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

template <typename T>
T* at(void* base, size_t off) {
  return off == kNone ? nullptr : (T*)((char*)base + off);
}
template <typename T>
const T* atc(const void* base, size_t off) {
  return off == kNone ? nullptr : (const T*)((const char*)base + off);
}

// the thread's last error message (dit_last_error) and the status that sets it
extern thread_local char g_err[512];
dit_status fail(dit_status st, const char* fmt, ...);
dit_status hip_check(hipError_t e, const char* what);

dit_status check_config(const dit_config* c);
dit_status check_sigmas(const dit_config* c, const double* sigmas, int n_sigmas);

// Byte offsets of the prepared weights of one configuration.
struct PrepLayout {
  size_t norm1 = kNone, norm2 = kNone, ln1_b = kNone, ln2_b = kNone, post_attn = kNone,
         post_ffn = kNone, w_qkv = kNone, w_out = kNone, w_fc1 = kNone, w_fc2 = kNone,
         b_qkv = kNone, b_out = kNone, b_fc1 = kNone, b_fc2 = kNone, q_norm = kNone,
         k_norm = kNone, basis = kNone, abias = kNone, table = kNone, tw1 = kNone, tb1 = kNone,
         tw2 = kNone, tb2 = kNone, aw = kNone, ab = kNone, rope_freq = kNone, total = 0;
};
PrepLayout prep_layout(const dit_config* c);
dit_ws_layout ws_layout(const dit_config* c, int n);

// Variant predicates and the modulation-row launch shared by the entry points.
bool has_mods(const dit_config* c);
bool temb_variant(const dit_config* c);
// Modulation rows into `mods` on stream s; `temb` is the timestep MLP's
// scratch ([temb_hidden + temb_freq] floats; Z-Image variants only).
dit_status launch_mods(const dit_config* c, const void* prep, const double* sigmas, float* mods,
                       float* temb, hipStream_t s);

// An output head (DIT_FINAL / DIT_ZFINAL) with its scale factor alpha.
dit_status final_forward_impl(const dit_config* c, const void* prepared, const float* h, int32_t n,
                              const int32_t* rows, const double* sigmas, int32_t n_sigmas, float alpha,
                              float* out, void* workspace, size_t ws_bytes, void* stream);

}  // namespace dit_host

#define DIT_TRY(expr)              \
  do {                             \
    dit_status st_ = (expr);       \
    if (st_ != DIT_OK) return st_; \
  } while (0)
#define HIP_TRY(expr, what) DIT_TRY(dit_host::hip_check((expr), what))
// Host-side exceptions (a failed allocation) never cross the C ABI: the entry
// points that allocate on the host end their body with this catch list.
#define DIT_CATCH_ALL                                                                  \
  catch (const std::bad_alloc&) {                                                      \
    return dit_host::fail(DIT_EINVAL, "host memory allocation failed");                \
  }                                                                                    \
  catch (...) {                                                                        \
    return dit_host::fail(DIT_EINVAL, "unexpected host exception");                    \
  }
