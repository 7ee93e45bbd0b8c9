// C ABI of libdit.so: host-side validation, buffer layouts and the launch
// sequence of one block on the caller's stream.  Validation touches no device
// memory and makes no HIP call, so every refusal can be exercised without a GPU.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "../../include/dit.h"
#include "dit_kernels.h"
#include "api_internal.h"

namespace dit_host {

thread_local char g_err[512] = "";

dit_status fail(dit_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}


size_t esize(const dit_config* c) { return c->dtype == DIT_BF16 ? 2 : 4; }
int chunks(const dit_config* c) {
  switch (c->variant) {
    case DIT_MMH3: return 6;
    case DIT_ZIMAGE: return 4;
    case DIT_FINAL: return 2;
    case DIT_ZFINAL: return 1;
    default: return 0;
  }
}
// rank-r basis variants: modulation rows from the interpolated timestep table
bool basis_mods(const dit_config* c) { return c->variant == DIT_MMH3 || c->variant == DIT_FINAL; }
// modulation rows from the sinusoidal timestep MLP (one row)
bool temb_variant(const dit_config* c) { return c->variant == DIT_ZIMAGE || c->variant == DIT_ZFINAL; }
// output heads, run by dit_final_forward
bool head(const dit_config* c) { return c->variant == DIT_FINAL || c->variant == DIT_ZFINAL; }
// Z-Image sandwich-norm blocks (modulated or not)
bool zsandwich(const dit_config* c) { return c->variant == DIT_ZIMAGE || c->variant == DIT_ZCONTEXT; }
int mod_rows(const dit_config* c) {
  return basis_mods(c) ? c->slots * c->tags : (temb_variant(c) ? 1 : 0);
}
bool swiglu(const dit_config* c) { return c->variant != DIT_SIGLIP; }
// modulated variants (adaLN rows, sigmas)
bool has_mods(const dit_config* c) { return basis_mods(c) || temb_variant(c); }
int fc1_rows(const dit_config* c) { return swiglu(c) ? 2 * c->F : c->F; }
// pair layout the kernels apply: the partial rotation runs as split-half over
// head dims permuted at weight preparation
int rope_pairs(const dit_config* c) { return c->rope == DIT_ROPE_PARTIAL ? DIT_ROPE_SPLIT_HALF : c->rope; }

dit_status check_config(const dit_config* c) {
  if (!c) return fail(DIT_EINVAL, "config is NULL");
  if (c->variant < DIT_MMH3 || c->variant > DIT_ZFINAL)
    return fail(DIT_EINVAL, "unknown variant %d", c->variant);
  if (c->dtype != DIT_F32 && c->dtype != DIT_BF16) return fail(DIT_EDTYPE, "unknown dtype %d", c->dtype);
  if (c->hd != 64 && c->hd != 128) return fail(DIT_EUNSUPPORTED, "head dim %d not in {64, 128}", c->hd);
  if (c->H <= 0 || c->D != c->H * c->hd) return fail(DIT_ESHAPE, "D=%d != H*hd=%d*%d", c->D, c->H, c->hd);
  if (c->D % 128 || c->D > 4096) return fail(DIT_EUNSUPPORTED, "D=%d must be a multiple of 128 and <= 4096", c->D);
  if (head(c)) {
    const int fm = c->dtype == DIT_BF16 ? 32 : 64;
    if (c->F <= 0 || c->F % fm) return fail(DIT_EUNSUPPORTED, "output width F=%d must be a positive multiple of %d", c->F, fm);
    if (c->variant == DIT_FINAL && c->tags != 1) return fail(DIT_EINVAL, "the final layer has one modality (tags=%d)", c->tags);
  } else if (c->F <= 0 || c->F % 128) {
    return fail(DIT_EUNSUPPORTED, "F=%d must be a positive multiple of 128", c->F);
  }
  if (!(c->eps >= 0.0f) || !(c->qk_eps >= 0.0f)) return fail(DIT_EINVAL, "eps must be >= 0");
  if (c->rope < DIT_ROPE_NONE || c->rope > DIT_ROPE_PARTIAL) return fail(DIT_EINVAL, "unknown rope %d", c->rope);
  if (c->rope == DIT_ROPE_PARTIAL) {
    if (c->variant != DIT_MMH3 && c->variant != DIT_REFINER)
      return fail(DIT_EUNSUPPORTED, "DIT_ROPE_PARTIAL is an MMH3 / refiner layout");
    const int d = c->rope_axes[0];
    if (d <= 0 || d % 2 || c->rope_axes[1] != d || c->rope_axes[2] != d)
      return fail(DIT_EINVAL, "DIT_ROPE_PARTIAL needs three equal, even, positive axis dims");
    if (3 * d > c->hd) return fail(DIT_ESHAPE, "DIT_ROPE_PARTIAL rotates 3 * %d dims, head dim is %d", d, c->hd);
  } else if (c->rope != DIT_ROPE_NONE && !head(c)) {
    int sum = 0;
    for (int a = 0; a < 3; ++a) {
      if (c->rope_axes[a] < 0 || c->rope_axes[a] % 2) return fail(DIT_EINVAL, "rope axis dims must be even and >= 0");
      sum += c->rope_axes[a];
    }
    if (sum != c->hd) return fail(DIT_ESHAPE, "rope axis dims sum to %d, head dim is %d", sum, c->hd);
    if (!(c->rope_theta > 0.0) || !isfinite(c->rope_theta)) return fail(DIT_EINVAL, "rope_theta must be > 0");
  }
  if (c->adaln_shared != 0 && (c->adaln_shared != 1 || !basis_mods(c)))
    return fail(DIT_EINVAL, "adaln_shared=%d (0, or 1 for MMH3 / FINAL)", c->adaln_shared);
  if (basis_mods(c)) {
    if (c->slots < 1 || c->slots > kMaxSlots) return fail(DIT_EUNSUPPORTED, "slots=%d not in [1, %d]", c->slots, kMaxSlots);
    if (c->tags < 1 || c->tags > 16) return fail(DIT_EINVAL, "tags=%d not in [1, 16]", c->tags);
    if (c->rank < 1 || c->rank > 64) return fail(DIT_EUNSUPPORTED, "rank=%d not in [1, 64]", c->rank);
    if (c->grid < 2) return fail(DIT_EINVAL, "grid=%d must be >= 2", c->grid);
  }
  if (c->variant == DIT_SIGLIP && c->rope != DIT_ROPE_NONE)
    return fail(DIT_EUNSUPPORTED, "the SigLIP layer takes no RoPE");
  if (temb_variant(c)) {
    if (c->temb_freq < 2 || c->temb_freq % 2 || c->temb_hidden < 1)
      return fail(DIT_EINVAL, "temb sizes freq=%d hidden=%d invalid", c->temb_freq, c->temb_hidden);
  }
  g_err[0] = 0;
  return DIT_OK;
}

// ---------------------------------------------------------------- layouts ----

PrepLayout prep_layout(const dit_config* c) {
  PrepLayout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  const size_t D = c->D, F = c->F, es = esize(c);
  if (c->variant == DIT_FINAL) {
    L.w_fc1 = take(F * D * es);
    L.norm1 = take(D * 4);
    L.b_fc1 = take(F * 4);
    size_t rows = (size_t)c->slots * c->tags * 2 * D;
    L.basis = take(rows * c->rank * 4);
    L.abias = take(rows * 4);
    L.table = take((size_t)c->grid * c->rank * 4);
    L.total = off;
    return L;
  }
  if (c->variant == DIT_ZFINAL) {
    L.w_fc1 = take(F * D * es);
    L.b_fc1 = take(F * 4);
    L.norm1 = take(D * 4);  // LayerNorm without affine: gain 1, bias 0
    L.ln1_b = take(D * 4);
    size_t tf = c->temb_freq, th = c->temb_hidden;
    L.tw1 = take(th * tf * 4);
    L.tb1 = take(th * 4);
    L.tw2 = take(tf * th * 4);
    L.tb2 = take(tf * 4);
    L.aw = take(D * tf * 4);
    L.ab = take(D * 4);
    L.total = off;
    return L;
  }
  L.w_qkv = take(3 * D * D * es);
  L.w_out = take(D * D * es);
  L.w_fc1 = take((size_t)fc1_rows(c) * D * es);
  L.w_fc2 = take(D * F * es);
  L.norm1 = take(D * 4);
  L.norm2 = take(D * 4);
  if (c->variant != DIT_SIGLIP) {
    L.q_norm = take(c->hd * 4);
    L.k_norm = take(c->hd * 4);
  }
  if (c->rope == DIT_ROPE_PARTIAL) L.rope_freq = take(c->rope_axes[0] / 2 * 4);
  if (c->variant == DIT_SIGLIP) {
    L.ln1_b = take(D * 4);
    L.ln2_b = take(D * 4);
    L.b_qkv = take(3 * D * 4);
    L.b_out = take(D * 4);
    L.b_fc1 = take(F * 4);
    L.b_fc2 = take(D * 4);
  }
  if (c->variant == DIT_MMH3) {
    size_t rows = (size_t)c->slots * c->tags * 6 * D;
    L.basis = take(rows * c->rank * 4);
    L.abias = take(rows * 4);
    L.table = take((size_t)c->grid * c->rank * 4);
  }
  if (zsandwich(c)) {
    L.post_attn = take(D * 4);
    L.post_ffn = take(D * 4);
  }
  if (c->variant == DIT_ZIMAGE) {
    size_t tf = c->temb_freq, th = c->temb_hidden;
    L.tw1 = take(th * tf * 4);
    L.tb1 = take(th * 4);
    L.tw2 = take(tf * th * 4);
    L.tb2 = take(tf * 4);
    L.aw = take(4 * D * tf * 4);
    L.ab = take(4 * D * 4);
  }
  L.total = off;
  return L;
}

int ldn_of(int n) { return (n + 127) / 128 * 128; }

dit_ws_layout ws_layout(const dit_config* c, int n) {
  dit_ws_layout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  const size_t D = c->D, F = c->F, es = esize(c);
  const int ldn = ldn_of(n);
  L.ldn = ldn;
  L.mods = mod_rows(c) ? take((size_t)mod_rows(c) * chunks(c) * D * 4) : kNone;
  if (head(c)) {  // a head: modulation rows (+ timestep MLP scratch) and the normalized rows only
    L.rope = L.qkv = L.q = L.k = L.vt = L.o = L.x1 = L.a = L.y = L.temb = L.part = kNone;
    if (c->variant == DIT_ZFINAL) L.temb = take((size_t)(c->temb_hidden + c->temb_freq) * 4);
    L.xn = take((size_t)n * D * es);
    L.total = off;
    return L;
  }
  L.temb = temb_variant(c) ? take((size_t)(c->temb_hidden + c->temb_freq) * 4) : kNone;
  L.rope = c->rope != DIT_ROPE_NONE ? take((size_t)n * (c->hd / 2) * 8) : kNone;
  L.xn = take((size_t)n * D * es);
  // the bf16 QKV GEMM writes q, k and v^T directly; only the fp32 path stages qkv
  L.qkv = c->dtype == DIT_F32 ? take((size_t)n * 3 * D * es) : kNone;
  L.q = take((size_t)c->H * ldn * c->hd * es);
  L.k = take((size_t)c->H * ldn * c->hd * es);
  L.vt = take((size_t)c->H * ldn * c->hd * es);
  L.o = take((size_t)n * D * es);
  L.x1 = take((size_t)n * D * 4);
  L.a = take((size_t)n * F * es);
  L.y = zsandwich(c) ? take((size_t)n * D * 4) : kNone;
  // attention's split key ranges and the GEMMs' split-K tails (never live at once)
  L.part = c->dtype == DIT_BF16
               ? take(std::max(dit::attention_part_bytes(c->hd), dit::gemm_split_bytes()))
               : kNone;
  L.total = off;
  return L;
}


dit_status hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(DIT_EHIP, "%s: %s", what, hipGetErrorString(e));
  return DIT_OK;
}


dit_status check_sigmas(const dit_config* c, const double* sigmas, int n_sigmas) {
  if (!has_mods(c)) return DIT_OK;
  int need = basis_mods(c) ? c->slots : 1;
  if (!sigmas) return fail(DIT_EINVAL, "sigmas is NULL");
  if (n_sigmas != need) return fail(DIT_ESHAPE, "n_sigmas=%d, the configuration needs %d", n_sigmas, need);
  for (int i = 0; i < need; ++i)
    if (!isfinite(sigmas[i])) return fail(DIT_EINVAL, "sigma %d is not finite", i);
  return DIT_OK;
}

// Modulation rows into `mods` (device).  MMH3: slot timestep t = 1 - sigma
// and grid coordinate p = clamp(t, 0, 1) * (G - 1), i0 = min(floor(p), G - 2),
// f = p - i0, all in fp64 ([MMH3] Adaln::eval; a slot at t = 1 reads table row
// G - 1 with weight 1).  The page floors only the video sigma, inside its
// forward and before the audio remap; dit_mmh3_slots applies that floor, so
// the slot sigmas are taken here as given.
dit_status launch_mods(const dit_config* c, const void* prep, const double* sigmas, float* mods,
                       float* temb, hipStream_t s) {
  PrepLayout P = prep_layout(c);
  if (basis_mods(c)) {
    dit::SlotCoords sc;
    memset(&sc, 0, sizeof(sc));
    for (int i = 0; i < c->slots; ++i) {
      double t = 1.0 - sigmas[i];
      double p = std::min(std::max(t, 0.0), 1.0) * (double)(c->grid - 1);
      int i0 = std::min((int)floor(p), c->grid - 2);
      sc.i0[i] = i0;
      sc.f[i] = (float)(p - (double)i0);
    }
    int per_slot = c->tags * chunks(c) * c->D;
    HIP_TRY(dit::adaln_interp(atc<float>(prep, P.basis), atc<float>(prep, P.abias),
                              atc<float>(prep, P.table), c->rank, per_slot, c->slots, sc, mods, s),
            "adaln_interp");
  } else if (temb_variant(c)) {
    // the final layer's adaLN reads silu(temb), the blocks' temb itself
    const bool fin = c->variant == DIT_ZFINAL;
    HIP_TRY(dit::temb_mods(sigmas[0] * (double)c->t_scale, c->temb_freq, c->temb_hidden, chunks(c) * c->D,
                           atc<float>(prep, P.tw1), atc<float>(prep, P.tb1), atc<float>(prep, P.tw2),
                           atc<float>(prep, P.tb2), atc<float>(prep, P.aw), atc<float>(prep, P.ab),
                           temb, mods, s, fin),
            "temb_mods");
  }
  return DIT_OK;
}

// Pre-norm (+ modulate) of one half into xn.
dit_status launch_prenorm(const dit_config* c, const void* prep, const float* x, int n,
                          const int* rows, const float* mods, int half, void* xn, hipStream_t s) {
  PrepLayout P = prep_layout(c);
  const int D = c->D;
  const bool bf = c->dtype == DIT_BF16;
  const float* g = atc<float>(prep, half ? P.norm2 : P.norm1);
  if (c->variant == DIT_MMH3) {
    HIP_TRY(dit::norm_mod(dit::NORM_RMS, dit::MOD_SHIFT_SCALE, bf, x, n, D, g, nullptr, c->eps, mods,
                          6 * D, rows, (half ? 3 : 0) * D, (half ? 4 : 1) * D, xn, s),
            "norm_mod");
  } else if (c->variant == DIT_ZIMAGE) {
    HIP_TRY(dit::norm_mod(dit::NORM_RMS, dit::MOD_SCALE, bf, x, n, D, g, nullptr, c->eps, mods, 4 * D,
                          nullptr, 0, (half ? 2 : 0) * D, xn, s),
            "norm_mod");
  } else if (c->variant == DIT_FINAL) {  // shift chunk 0, scale chunk 1 of the token's slot
    HIP_TRY(dit::norm_mod(dit::NORM_RMS, dit::MOD_SHIFT_SCALE, bf, x, n, D, g, nullptr, c->eps, mods,
                          2 * D, rows, 0, D, xn, s),
            "norm_mod");
  } else if (c->variant == DIT_ZFINAL) {  // LayerNorm without affine (gain 1, bias 0), * (1 + scale)
    HIP_TRY(dit::norm_mod(dit::NORM_LAYER, dit::MOD_SCALE, bf, x, n, D, g, atc<float>(prep, P.ln1_b), c->eps,
                          mods, D, nullptr, 0, 0, xn, s),
            "norm_mod");
  } else if (c->variant == DIT_REFINER || c->variant == DIT_ZCONTEXT) {
    HIP_TRY(dit::norm_mod(dit::NORM_RMS, dit::MOD_NONE, bf, x, n, D, g, nullptr, c->eps, nullptr, 0,
                          nullptr, 0, 0, xn, s),
            "norm_mod");
  } else {
    HIP_TRY(dit::norm_mod(dit::NORM_LAYER, dit::MOD_NONE, bf, x, n, D, g,
                          atc<float>(prep, half ? P.ln2_b : P.ln1_b), c->eps, nullptr, 0, nullptr, 0,
                          0, xn, s),
            "norm_mod");
  }
  return DIT_OK;
}

// Per-phase event timing (thread-local; see dit_profile_begin).
struct Profiler {
  bool on = false;
  int max_calls = 0, used = 0;
  std::vector<hipEvent_t> ev;
};
thread_local Profiler g_prof;

struct PhaseMarks {
  hipStream_t s;
  hipEvent_t* ev = nullptr;
  explicit PhaseMarks(hipStream_t st) : s(st) {
    if (g_prof.on && g_prof.used < g_prof.max_calls) {
      ev = &g_prof.ev[(size_t)g_prof.used * (DIT_NPHASES + 1)];
      ++g_prof.used;
      (void)hipEventRecord(ev[0], s);
    }
  }
  void mark(int phase) {
    if (ev) (void)hipEventRecord(ev[phase + 1], s);
  }
};

const char* kPhaseNames[DIT_NPHASES] = {"adaln+rope", "norm1", "qkv_gemm", "qk_split", "attention",
                                        "out_gemm", "norm2", "fc1_gemm", "fc2_gemm"};

}  // namespace dit_host

using namespace dit_host;

extern "C" {

const char* dit_phase_name(int32_t phase) {
  return (phase >= 0 && phase < DIT_NPHASES) ? kPhaseNames[phase] : "";
}

dit_status dit_profile_begin(int32_t max_calls) {
  if (max_calls < 1 || max_calls > 100000) return fail(DIT_EINVAL, "max_calls=%d not in [1, 100000]", max_calls);
  if (g_prof.on) return fail(DIT_EINVAL, "profiling already armed on this thread");
  try {
    g_prof.ev.assign((size_t)max_calls * (DIT_NPHASES + 1), nullptr);
  } DIT_CATCH_ALL
  for (auto& e : g_prof.ev) {
    hipError_t err = hipEventCreate(&e);
    if (err != hipSuccess) {
      for (auto& f : g_prof.ev)
        if (f) (void)hipEventDestroy(f);
      g_prof.ev.clear();
      return hip_check(err, "hipEventCreate");
    }
  }
  g_prof.on = true;
  g_prof.max_calls = max_calls;
  g_prof.used = 0;
  return DIT_OK;
}

dit_status dit_profile_end(double* phase_ms, int32_t* calls) {
  if (!g_prof.on) return fail(DIT_EINVAL, "profiling is not armed");
  if (!phase_ms || !calls) return fail(DIT_EINVAL, "phase_ms/calls is NULL");
  dit_status st = DIT_OK;
  for (int p = 0; p < DIT_NPHASES; ++p) phase_ms[p] = 0.0;
  if (g_prof.used > 0) {
    hipError_t e = hipEventSynchronize(g_prof.ev[(size_t)g_prof.used * (DIT_NPHASES + 1) - 1]);
    if (e != hipSuccess) st = hip_check(e, "hipEventSynchronize");
    for (int c = 0; c < g_prof.used && st == DIT_OK; ++c)
      for (int p = 0; p < DIT_NPHASES; ++p) {
        float ms = 0.0f;
        hipError_t e2 = hipEventElapsedTime(&ms, g_prof.ev[(size_t)c * (DIT_NPHASES + 1) + p],
                                            g_prof.ev[(size_t)c * (DIT_NPHASES + 1) + p + 1]);
        if (e2 != hipSuccess) {
          st = hip_check(e2, "hipEventElapsedTime");
          break;
        }
        phase_ms[p] += ms;
      }
  }
  *calls = g_prof.used;
  for (auto& e : g_prof.ev) (void)hipEventDestroy(e);
  g_prof.ev.clear();
  g_prof.on = false;
  g_prof.used = g_prof.max_calls = 0;
  return st;
}


int32_t dit_abi_version(void) { return 7; }

const char* dit_last_error(void) { return g_err; }

double dit_sigma_remap(double sigma, double from_shift, double to_shift) {
  // Base-grid point of sigma on the from_shift schedule, then onto to_shift's
  // ([MMH3] time_shift_sigma).
  double base = sigma / (from_shift + sigma * (1.0 - from_shift));
  return to_shift * base / (1.0 + (to_shift - 1.0) * base);
}

double dit_sigma_remap_slope(double sigma, double from_shift, double to_shift) {
  double base = sigma / (from_shift + sigma * (1.0 - from_shift));
  double a = 1.0 + (from_shift - 1.0) * base, b = 1.0 + (to_shift - 1.0) * base;
  return (to_shift * a * a) / (from_shift * b * b);
}

dit_status dit_validate_config(const dit_config* cfg) { return check_config(cfg); }

size_t dit_prepared_size(const dit_config* cfg) {
  if (check_config(cfg) != DIT_OK) return 0;
  return prep_layout(cfg).total;
}

size_t dit_workspace_size(const dit_config* cfg, int32_t n) {
  if (check_config(cfg) != DIT_OK || bad_tokens(n)) return 0;
  return ws_layout(cfg, n).total;
}

dit_status dit_workspace_layout(const dit_config* cfg, int32_t n, dit_ws_layout* out) {
  DIT_TRY(check_config(cfg));
  if (bad_tokens(n)) return fail(DIT_ESHAPE, "n=%d not in [0, %d]", n, kMaxTokens);
  if (!out) return fail(DIT_EINVAL, "out is NULL");
  *out = ws_layout(cfg, n);
  return DIT_OK;
}

dit_status dit_prepare_weights(const dit_config* c, const dit_weights* w, void* prepared,
                               size_t bytes, void* stream) {
  DIT_TRY(check_config(c));
  if (!w) return fail(DIT_EINVAL, "weights is NULL");
  if (!prepared) return fail(DIT_EINVAL, "prepared is NULL");
  if ((uintptr_t)prepared % kAlign) return fail(DIT_EALIGN, "prepared must be 256-byte aligned");
  PrepLayout P = prep_layout(c);
  if (bytes < P.total) return fail(DIT_EWORKSPACE, "prepared buffer %zu < %zu bytes", bytes, P.total);
  struct Need {
    const void* p;
    const char* name;
  };
  hipStream_t s = (hipStream_t)stream;
  if (c->variant == DIT_FINAL) {
    Need need[] = {{w->norm1, "norm1"}, {w->w_fc1, "w_fc1 (head)"}, {w->adaln_basis, "adaln_basis"},
                   {w->adaln_table, "adaln_table"}};
    for (auto& q : need) {
      if (!q.p) return fail(DIT_EINVAL, "weight %s is NULL", q.name);
      if (!aligned16(q.p)) return fail(DIT_EALIGN, "weight %s is not 16-byte aligned", q.name);
    }
    const int D = c->D, F = c->F, rows = c->slots * c->tags * 2 * D;
    HIP_TRY(dit::prep_matrix(c->dtype, w->w_fc1, at<char>(prepared, P.w_fc1), F, D, 0, 0, 1.0f, s), "prep head");
    HIP_TRY(dit::prep_vector(w->norm1, at<float>(prepared, P.norm1), D, 0, 1.0f, s), "prep norm1");
    HIP_TRY(dit::prep_vector(w->b_fc1, at<float>(prepared, P.b_fc1), F, 0, 1.0f, s), "prep head bias");
    dit::RowMap am;
    am.src_mod = c->adaln_shared ? c->tags * 2 * D : 0;
    HIP_TRY(dit::prep_matrix(dit::F32, w->adaln_basis, at<char>(prepared, P.basis), rows, c->rank, am, 0, 1.0f, s),
            "prep adaln_basis");
    HIP_TRY(dit::prep_vector(w->adaln_bias, at<float>(prepared, P.abias), rows, am, 0, 1.0f, s), "prep adaln_bias");
    HIP_TRY(dit::prep_matrix(dit::F32, w->adaln_table, at<char>(prepared, P.table), c->grid, c->rank, 0, 0, 1.0f, s),
            "prep adaln_table");
    return DIT_OK;
  }
  if (c->variant == DIT_ZFINAL) {
    Need need[] = {{w->w_fc1, "w_fc1 (output)"}, {w->temb_w1, "temb_w1"}, {w->temb_w2, "temb_w2"},
                   {w->ada_w, "ada_w"}};
    for (auto& q : need) {
      if (!q.p) return fail(DIT_EINVAL, "weight %s is NULL", q.name);
      if (!aligned16(q.p)) return fail(DIT_EALIGN, "weight %s is not 16-byte aligned", q.name);
    }
    const int D = c->D, F = c->F, tf = c->temb_freq, th = c->temb_hidden;
    HIP_TRY(dit::prep_matrix(c->dtype, w->w_fc1, at<char>(prepared, P.w_fc1), F, D, 0, 0, 1.0f, s), "prep output");
    HIP_TRY(dit::prep_vector(w->b_fc1, at<float>(prepared, P.b_fc1), F, 0, 1.0f, s), "prep output bias");
    HIP_TRY(dit::fill_f32(at<float>(prepared, P.norm1), D, 1.0f, s), "norm gain");
    HIP_TRY(dit::prep_vector(nullptr, at<float>(prepared, P.ln1_b), D, 0, 1.0f, s), "norm bias");
    HIP_TRY(dit::prep_matrix(dit::F32, w->temb_w1, at<char>(prepared, P.tw1), th, tf, 0, 0, 1.0f, s), "prep temb_w1");
    HIP_TRY(dit::prep_vector(w->temb_b1, at<float>(prepared, P.tb1), th, 0, 1.0f, s), "prep temb_b1");
    HIP_TRY(dit::prep_matrix(dit::F32, w->temb_w2, at<char>(prepared, P.tw2), tf, th, 0, 0, 1.0f, s), "prep temb_w2");
    HIP_TRY(dit::prep_vector(w->temb_b2, at<float>(prepared, P.tb2), tf, 0, 1.0f, s), "prep temb_b2");
    HIP_TRY(dit::prep_matrix(dit::F32, w->ada_w, at<char>(prepared, P.aw), D, tf, 0, 0, 1.0f, s), "prep ada_w");
    HIP_TRY(dit::prep_vector(w->ada_b, at<float>(prepared, P.ab), D, 0, 1.0f, s), "prep ada_b");
    return DIT_OK;
  }
  Need common[] = {{w->w_qkv, "w_qkv"}, {w->w_out, "w_out"}, {w->w_fc1, "w_fc1"},
                   {w->w_fc2, "w_fc2"}, {w->norm1, "norm1"}, {w->norm2, "norm2"}};
  for (auto& q : common) {
    if (!q.p) return fail(DIT_EINVAL, "weight %s is NULL", q.name);
    if (!aligned16(q.p)) return fail(DIT_EALIGN, "weight %s is not 16-byte aligned", q.name);
  }
  if (c->variant != DIT_SIGLIP && (!w->q_norm || !w->k_norm)) return fail(DIT_EINVAL, "q_norm/k_norm are NULL");
  if (c->rope == DIT_ROPE_PARTIAL && !w->rope_freq) return fail(DIT_EINVAL, "rope_freq is NULL (DIT_ROPE_PARTIAL)");
  if (c->variant == DIT_MMH3 && (!w->adaln_basis || !w->adaln_table))
    return fail(DIT_EINVAL, "adaln_basis/adaln_table are NULL");
  if (c->variant == DIT_SIGLIP && (!w->ln1_b || !w->ln2_b))
    return fail(DIT_EINVAL, "SigLIP LayerNorm biases are NULL");
  if (c->variant == DIT_ZIMAGE &&
      (!w->post_attn_norm || !w->post_ffn_norm || !w->temb_w1 || !w->temb_w2 || !w->ada_w))
    return fail(DIT_EINVAL, "Z-Image norms or timestep weights are NULL");
  if (c->variant == DIT_ZCONTEXT && (!w->post_attn_norm || !w->post_ffn_norm))
    return fail(DIT_EINVAL, "Z-Image sandwich norms are NULL");

  const int D = c->D, F = c->F, dt = c->dtype;
  // [SIGLIP] Layer::load folds hd^-1/2 into W_q and b_q.
  const bool fold = c->variant == DIT_SIGLIP;
  const float qs = fold ? (float)(1.0 / sqrt((double)c->hd)) : 1.0f;
  dit::RowMap qkmap;  // partial RoPE: permute the head dims of the q and k rows
  if (c->rope == DIT_ROPE_PARTIAL) {
    qkmap.perm_rows = 2 * D;
    qkmap.perm_hd = c->hd;
    qkmap.perm_P = 3 * (c->rope_axes[0] / 2);
  }
  HIP_TRY(dit::prep_matrix(dt, w->w_qkv, at<char>(prepared, P.w_qkv), 3 * D, D, qkmap, fold ? D : 0, qs, s),
          "prep w_qkv");
  HIP_TRY(dit::prep_matrix(dt, w->w_out, at<char>(prepared, P.w_out), D, D, 0, 0, 1.0f, s), "prep w_out");
  HIP_TRY(dit::prep_matrix(dt, w->w_fc1, at<char>(prepared, P.w_fc1), fc1_rows(c), D,
                           swiglu(c) ? F : 0, 0, 1.0f, s), "prep w_fc1");
  HIP_TRY(dit::prep_matrix(dt, w->w_fc2, at<char>(prepared, P.w_fc2), D, F, 0, 0, 1.0f, s), "prep w_fc2");
  auto vec = [&](const float* src, size_t off, int n, int scale_n = 0, float sc = 1.0f) {
    return dit::prep_vector(src, at<float>(prepared, off), n, scale_n, sc, s);
  };
  HIP_TRY(vec(w->norm1, P.norm1, D), "prep norm1");
  HIP_TRY(vec(w->norm2, P.norm2, D), "prep norm2");
  if (c->variant != DIT_SIGLIP) {
    dit::RowMap gmap = qkmap;
    gmap.perm_rows = gmap.perm_rows ? c->hd : 0;
    HIP_TRY(dit::prep_vector(w->q_norm, at<float>(prepared, P.q_norm), c->hd, gmap, 0, 1.0f, s), "prep q_norm");
    HIP_TRY(dit::prep_vector(w->k_norm, at<float>(prepared, P.k_norm), c->hd, gmap, 0, 1.0f, s), "prep k_norm");
  }
  if (c->rope == DIT_ROPE_PARTIAL)
    HIP_TRY(vec(w->rope_freq, P.rope_freq, c->rope_axes[0] / 2), "prep rope_freq");
  if (c->variant == DIT_SIGLIP) {
    HIP_TRY(vec(w->ln1_b, P.ln1_b, D), "prep ln1_b");
    HIP_TRY(vec(w->ln2_b, P.ln2_b, D), "prep ln2_b");
    HIP_TRY(vec(w->b_qkv, P.b_qkv, 3 * D, D, qs), "prep b_qkv");
    HIP_TRY(vec(w->b_out, P.b_out, D), "prep b_out");
    HIP_TRY(vec(w->b_fc1, P.b_fc1, F), "prep b_fc1");
    HIP_TRY(vec(w->b_fc2, P.b_fc2, D), "prep b_fc2");
  }
  if (c->variant == DIT_MMH3) {
    int rows = c->slots * c->tags * 6 * D;
    dit::RowMap am;  // a shared basis is one slot's rows, repeated for every slot
    am.src_mod = c->adaln_shared ? c->tags * 6 * D : 0;
    HIP_TRY(dit::prep_matrix(dit::F32, w->adaln_basis, at<char>(prepared, P.basis), rows, c->rank, am, 0, 1.0f, s),
            "prep adaln_basis");
    HIP_TRY(dit::prep_vector(w->adaln_bias, at<float>(prepared, P.abias), rows, am, 0, 1.0f, s), "prep adaln_bias");
    HIP_TRY(dit::prep_matrix(dit::F32, w->adaln_table, at<char>(prepared, P.table), c->grid, c->rank, 0, 0, 1.0f, s),
            "prep adaln_table");
  }
  if (zsandwich(c)) {
    HIP_TRY(vec(w->post_attn_norm, P.post_attn, D), "prep post_attn_norm");
    HIP_TRY(vec(w->post_ffn_norm, P.post_ffn, D), "prep post_ffn_norm");
  }
  if (c->variant == DIT_ZIMAGE) {
    const int tf = c->temb_freq, th = c->temb_hidden;
    HIP_TRY(dit::prep_matrix(dit::F32, w->temb_w1, at<char>(prepared, P.tw1), th, tf, 0, 0, 1.0f, s), "prep temb_w1");
    HIP_TRY(vec(w->temb_b1, P.tb1, th), "prep temb_b1");
    HIP_TRY(dit::prep_matrix(dit::F32, w->temb_w2, at<char>(prepared, P.tw2), tf, th, 0, 0, 1.0f, s), "prep temb_w2");
    HIP_TRY(vec(w->temb_b2, P.tb2, tf), "prep temb_b2");
    HIP_TRY(dit::prep_matrix(dit::F32, w->ada_w, at<char>(prepared, P.aw), 4 * D, tf, 0, 0, 1.0f, s), "prep ada_w");
    HIP_TRY(vec(w->ada_b, P.ab, 4 * D), "prep ada_b");
  }
  return DIT_OK;
}

dit_status dit_adaln_eval(const dit_config* c, const void* prepared, const double* sigmas,
                          int32_t n_sigmas, float* mods_out, float* temb_scratch, void* stream) {
  DIT_TRY(check_config(c));
  if (!has_mods(c)) return fail(DIT_EUNSUPPORTED, "variant %d has no modulation", c->variant);
  if (!prepared || !mods_out) return fail(DIT_EINVAL, "prepared/mods_out is NULL");
  if (temb_variant(c) && !temb_scratch) return fail(DIT_EINVAL, "temb_scratch is NULL");
  DIT_TRY(check_sigmas(c, sigmas, n_sigmas));
  return launch_mods(c, prepared, sigmas, mods_out, temb_scratch, (hipStream_t)stream);
}

dit_status dit_adaln_modulate(const dit_config* c, const void* prepared, const float* x, int32_t n,
                              const int32_t* rows, const double* sigmas, int32_t n_sigmas,
                              int32_t half, void* xn_out, float* mods_out, float* temb_scratch,
                              void* stream) {
  DIT_TRY(check_config(c));
  if (bad_tokens(n)) return fail(DIT_ESHAPE, "n=%d not in [0, %d]", n, kMaxTokens);
  if (half != 0 && half != 1) return fail(DIT_EINVAL, "half=%d not in {0, 1}", half);
  if (!prepared) return fail(DIT_EINVAL, "prepared is NULL");
  if (has_mods(c)) {
    if (!mods_out) return fail(DIT_EINVAL, "mods_out is NULL");
    if (temb_variant(c) && !temb_scratch) return fail(DIT_EINVAL, "temb_scratch is NULL");
    DIT_TRY(check_sigmas(c, sigmas, n_sigmas));
  }
  if (n == 0) return DIT_OK;
  if (!x || !xn_out) return fail(DIT_EINVAL, "x/xn_out is NULL");
  if (!aligned16(x) || !aligned16(xn_out)) return fail(DIT_EALIGN, "x/xn_out not 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  if (has_mods(c)) DIT_TRY(launch_mods(c, prepared, sigmas, mods_out, temb_scratch, s));
  return launch_prenorm(c, prepared, x, n, rows, mods_out, half, xn_out, s);
}

// Host-side check of a packed-sample table: 1 <= nseq <= DIT_MAX_SEQS,
// starts[0] = 0, non-decreasing, starts[nseq] = n.
static dit_status check_seqs(const int32_t* seq_starts, int32_t nseq, int32_t n) {
  if (!seq_starts) return fail(DIT_EINVAL, "seq_starts is NULL");
  if (nseq < 1 || nseq > DIT_MAX_SEQS)
    return fail(DIT_ESHAPE, "nseq=%d outside [1, %d]", nseq, DIT_MAX_SEQS);
  if (seq_starts[0] != 0) return fail(DIT_ESHAPE, "seq_starts[0]=%d, must be 0", seq_starts[0]);
  for (int i = 0; i < nseq; ++i)
    if (seq_starts[i + 1] < seq_starts[i])
      return fail(DIT_ESHAPE, "seq_starts decreases at %d (%d -> %d)", i, seq_starts[i], seq_starts[i + 1]);
  if (seq_starts[nseq] != n)
    return fail(DIT_ESHAPE, "seq_starts[nseq]=%d must equal n=%d", seq_starts[nseq], n);
  return DIT_OK;
}

static dit_status attention_impl(const dit_config* c, const void* q, const void* k, const void* vt,
                          int32_t n, int32_t ldn, const int32_t* seq_starts, int32_t nseq,
                          float score_scale, void* o, void* stream) {
  DIT_TRY(check_config(c));
  if (bad_tokens(n) || ldn < n || ldn % 128 || bad_tokens(ldn))
    return fail(DIT_ESHAPE, "need 0 <= n <= ldn <= %d, ldn %% 128 == 0 (n=%d ldn=%d)", kMaxTokens, n, ldn);
  if (seq_starts) DIT_TRY(check_seqs(seq_starts, nseq, n));
  if (n == 0) return DIT_OK;
  if (!q || !k || !vt || !o) return fail(DIT_EINVAL, "q/k/vt/o is NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(vt) || !aligned16(o))
    return fail(DIT_EALIGN, "q/k/vt/o not 16-byte aligned");
  if (!isfinite(score_scale)) return fail(DIT_EINVAL, "score_scale not finite");
  const float log2e = 1.4426950408889634f;
  dit::SeqTable tab;
  dit::make_seq_table(seq_starts, nseq, n, &tab);
  HIP_TRY(dit::attention(c->dtype, c->hd, q, ldn, k, vt, n, ldn, c->H, score_scale * log2e, o,
                         nullptr, tab, (hipStream_t)stream),
          "attention");
  return DIT_OK;
}

dit_status dit_attention(const dit_config* c, const void* q, const void* k, const void* vt,
                         int32_t n, int32_t ldn, float score_scale, void* o, void* stream) {
  return attention_impl(c, q, k, vt, n, ldn, nullptr, 0, score_scale, o, stream);
}

dit_status dit_attention_packed(const dit_config* c, const void* q, const void* k, const void* vt,
                                int32_t n, int32_t ldn, const int32_t* seq_starts, int32_t nseq,
                                float score_scale, void* o, void* stream) {
  if (!seq_starts) return fail(DIT_EINVAL, "seq_starts is NULL");
  return attention_impl(c, q, k, vt, n, ldn, seq_starts, nseq, score_scale, o, stream);
}

size_t dit_attention_shard_workspace_size(const dit_config* c) {
  if (check_config(c) != DIT_OK) return 0;
  return c->dtype == DIT_BF16 ? dit::attention_part_bytes(c->hd) : 0;
}

dit_status dit_attention_shard(const dit_config* c, const void* q, int32_t ldq, int32_t qlo,
                               int32_t qhi, const void* k, const void* vt, int32_t n, int32_t ldn,
                               float score_scale, void* o, void* workspace, size_t ws_bytes,
                               void* stream) {
  DIT_TRY(check_config(c));
  if (bad_tokens(n) || ldn < n || ldn % 128 || bad_tokens(ldn))
    return fail(DIT_ESHAPE, "need 0 <= n <= ldn <= %d, ldn %% 128 == 0 (n=%d ldn=%d)", kMaxTokens, n, ldn);
  if (qlo < 0 || qhi < qlo || qhi > n)
    return fail(DIT_ESHAPE, "need 0 <= qlo <= qhi <= n (qlo=%d qhi=%d n=%d)", qlo, qhi, n);
  if (ldq < qhi - qlo || ldq % 128 || bad_tokens(ldq))
    return fail(DIT_ESHAPE, "need qhi - qlo <= ldq <= %d, ldq %% 128 == 0 (ldq=%d)", kMaxTokens, ldq);
  if (qhi == qlo) return DIT_OK;
  if (!q || !k || !vt || !o) return fail(DIT_EINVAL, "q/k/vt/o is NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(vt) || !aligned16(o))
    return fail(DIT_EALIGN, "q/k/vt/o not 16-byte aligned");
  if (!isfinite(score_scale)) return fail(DIT_EINVAL, "score_scale not finite");
  const size_t need = dit_attention_shard_workspace_size(c);
  if (need && (!workspace || ws_bytes < need))
    return fail(DIT_EWORKSPACE, "workspace %zu < %zu bytes", workspace ? ws_bytes : (size_t)0, need);
  if (need && (uintptr_t)workspace % kAlign) return fail(DIT_EALIGN, "workspace must be 256-byte aligned");
  const float log2e = 1.4426950408889634f;
  dit::SeqTable tab;
  dit::make_shard_table(n, qlo, qhi, &tab);
  HIP_TRY(dit::attention(c->dtype, c->hd, q, ldq, k, vt, n, ldn, c->H, score_scale * log2e, o,
                         need ? (float*)workspace : nullptr, tab, (hipStream_t)stream),
          "attention shard");
  return DIT_OK;
}

// mods_in: modulation rows supplied by the caller (skips their evaluation).
static dit_status block_forward_impl(const dit_config* c, const void* prepared, const float* x, int32_t n,
                              const int32_t* rows, const float* pos, const double* sigmas,
                              int32_t n_sigmas, const float* mods_in, const int32_t* seq_starts,
                              int32_t nseq, float* out, void* workspace, size_t ws_bytes,
                              void* stream) {
  DIT_TRY(check_config(c));
  if (head(c)) return fail(DIT_EUNSUPPORTED, "output heads are run by dit_final_forward");
  if (bad_tokens(n)) return fail(DIT_ESHAPE, "n=%d not in [0, %d]", n, kMaxTokens);
  if (seq_starts) DIT_TRY(check_seqs(seq_starts, nseq, n));
  if (!prepared) return fail(DIT_EINVAL, "prepared is NULL");
  if (mods_in) {
    if (!has_mods(c)) return fail(DIT_EUNSUPPORTED, "variant %d has no modulation", c->variant);
    if (!aligned16(mods_in)) return fail(DIT_EALIGN, "mods not 16-byte aligned");
  } else {
    DIT_TRY(check_sigmas(c, sigmas, n_sigmas));
  }
  if (n == 0) return DIT_OK;
  if (!x || !out) return fail(DIT_EINVAL, "x/out is NULL");
  if (!aligned16(x) || !aligned16(out)) return fail(DIT_EALIGN, "x/out not 16-byte aligned");
  if (c->rope != DIT_ROPE_NONE && !pos) return fail(DIT_EINVAL, "pos is NULL but the block applies RoPE");
  if (!workspace) return fail(DIT_EINVAL, "workspace is NULL");
  if ((uintptr_t)workspace % kAlign) return fail(DIT_EALIGN, "workspace must be 256-byte aligned");
  dit_ws_layout L = ws_layout(c, n);
  if (ws_bytes < L.total) return fail(DIT_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, L.total);

  hipStream_t s = (hipStream_t)stream;
  PrepLayout P = prep_layout(c);
  const int D = c->D, F = c->F, H = c->H, hd = c->hd, dt = c->dtype;
  const bool bf = dt == DIT_BF16;
  const int ldn = L.ldn;
  const float* mods = mods_in ? mods_in : at<float>(workspace, L.mods);
  void* xn = at<char>(workspace, L.xn);
  void* qkv = at<char>(workspace, L.qkv);
  void* q = at<char>(workspace, L.q);
  void* k = at<char>(workspace, L.k);
  void* vt = at<char>(workspace, L.vt);
  void* o = at<char>(workspace, L.o);
  float* x1 = at<float>(workspace, L.x1);
  void* a = at<char>(workspace, L.a);
  float* y = at<float>(workspace, L.y);
  float* cs = at<float>(workspace, L.rope);

  PhaseMarks pm(s);
  // a1: modulation rows; RoPE table
  if (has_mods(c) && !mods_in)
    DIT_TRY(launch_mods(c, prepared, sigmas, at<float>(workspace, L.mods), at<float>(workspace, L.temb), s));
  if (c->rope == DIT_ROPE_PARTIAL)
    HIP_TRY(dit::rope_table_shared(pos, n, hd / 2, c->rope_axes[0] / 2, atc<float>(prepared, P.rope_freq), cs, s),
            "rope_table");
  else if (c->rope != DIT_ROPE_NONE)
    HIP_TRY(dit::rope_table(pos, n, hd / 2, c->rope_axes, c->rope_theta, cs, s), "rope_table");
  pm.mark(0);
  // a2: pre-norm + modulate
  DIT_TRY(launch_prenorm(c, prepared, x, n, rows, mods, 0, xn, s));
  pm.mark(1);
  float* const gsplit = bf ? at<float>(workspace, L.part) : nullptr;  // split-K tails
  // a3 + a4: QKV projection (+ bias), qk-norm, RoPE and the score-scale fold into q,
  // head-major q and k and transposed v (fused into the GEMM epilogue for bf16)
  {
    const bool qkn = c->variant != DIT_SIGLIP;
    // q carries the whole base-2 score scale, log2(e) * hd^-1/2 (SigLIP's
    // hd^-1/2 is already in W_q), so the attention kernel runs with scale 1.
    const double kLog2e = 1.4426950408889634;
    const float q_scale =
        (float)(kLog2e * (c->variant == DIT_SIGLIP ? 1.0 : 1.0 / sqrt((double)hd)));
    const float* qn = qkn ? atc<float>(prepared, P.q_norm) : nullptr;
    const float* kn = qkn ? atc<float>(prepared, P.k_norm) : nullptr;
    dit::Epi ep;
    ep.split = gsplit;
    ep.bias = atc<float>(prepared, P.b_qkv);
    if (bf) {
      ep.ldc = D;
      ep.hd = hd;
      ep.ldn = ldn;
      ep.qn = qn;
      ep.kn = kn;
      ep.qk_eps = c->qk_eps;
      ep.cs = cs;
      ep.rope = rope_pairs(c);
      ep.q_scale = q_scale;
      ep.q = q;
      ep.k = k;
      ep.vt = vt;
      HIP_TRY(dit::gemm(dt, dit::EPI_QKV, true, xn, D, atc<char>(prepared, P.w_qkv), D, n, 3 * D, D, ep, s),
              "qkv gemm");
      pm.mark(2);
    } else {
      ep.out = qkv;
      ep.ldc = 3 * D;
      HIP_TRY(dit::gemm(dt, dit::EPI_STORE, false, xn, D, atc<char>(prepared, P.w_qkv), D, n, 3 * D, D, ep, s),
              "qkv gemm");
      pm.mark(2);
      HIP_TRY(dit::qk_split(dt, hd, qkv, n, ldn, H, qn, kn, c->qk_eps, cs, rope_pairs(c), q_scale, q, k, vt, s),
              "qk_split");
    }
  }
  pm.mark(3);
  // a5: attention (q carries log2(e) hd^-1/2; the kernel works in base 2)
  {
    dit::SeqTable tab;
    dit::make_seq_table(seq_starts, nseq, n, &tab);
    HIP_TRY(dit::attention(dt, hd, q, ldn, k, vt, n, ldn, H, 1.0f, o,
                           bf ? at<float>(workspace, L.part) : nullptr, tab, s),
            "attention");
  }
  pm.mark(4);
  // a6: out projection + residual
  // Z-Image chunks (scale_msa, gate_msa, scale_mlp, gate_mlp); none for the context refiner
  auto zmod = [&](int e) -> const float* { return c->variant == DIT_ZIMAGE ? mods + e * D : nullptr; };
  if (zsandwich(c)) {
    dit::Epi ep;
    ep.split = gsplit;
    ep.out = y;
    ep.ldc = D;
    HIP_TRY(dit::gemm(dt, dit::EPI_STORE, false, o, D, atc<char>(prepared, P.w_out), D, n, D, D, ep, s), "out gemm");
    // x1 = x + tanh(gate_msa) RMSNorm(y); xn = RMSNorm(x1) (1 + scale_mlp)
    HIP_TRY(dit::sandwich(x, y, n, D, atc<float>(prepared, P.post_attn), zmod(1), c->eps, x1,
                          atc<float>(prepared, P.norm2), zmod(2), bf, xn, s),
            "sandwich attn");
    pm.mark(5);
    pm.mark(6);
  } else {
    dit::Epi ep;
    ep.split = gsplit;
    ep.out = x1;
    ep.ldc = D;
    ep.resid = x;
    ep.ldr = D;
    ep.bias = atc<float>(prepared, P.b_out);
    if (c->variant == DIT_MMH3) {
      ep.mods = mods;
      ep.mstride = 6 * D;
      ep.goff = 2 * D;
      ep.rows = rows;
    }
    HIP_TRY(dit::gemm(dt, dit::EPI_GATED_RES, false, o, D, atc<char>(prepared, P.w_out), D, n, D, D, ep, s),
            "out gemm");
    pm.mark(5);
    // a7: FFN pre-norm + modulate
    DIT_TRY(launch_prenorm(c, prepared, x1, n, rows, mods, 1, xn, s));
    pm.mark(6);
  }
  // a8: fc1 + activation
  {
    dit::Epi ep;
    ep.split = gsplit;
    ep.out = a;
    ep.ldc = F;
    ep.bias = atc<float>(prepared, P.b_fc1);
    HIP_TRY(dit::gemm(dt, swiglu(c) ? dit::EPI_SWIGLU : dit::EPI_GELU, bf, xn, D, atc<char>(prepared, P.w_fc1), D, n,
                      fc1_rows(c), D, ep, s),
            "fc1 gemm");
  }
  pm.mark(7);
  // a9: fc2 + residual
  if (zsandwich(c)) {
    dit::Epi ep;
    ep.split = gsplit;
    ep.out = y;
    ep.ldc = D;
    HIP_TRY(dit::gemm(dt, dit::EPI_STORE, false, a, F, atc<char>(prepared, P.w_fc2), F, n, D, F, ep, s), "fc2 gemm");
    HIP_TRY(dit::sandwich(x1, y, n, D, atc<float>(prepared, P.post_ffn), zmod(3), c->eps, out, nullptr,
                          nullptr, bf, nullptr, s),
            "sandwich ffn");
  } else {
    dit::Epi ep;
    ep.split = gsplit;
    ep.out = out;
    ep.ldc = D;
    ep.resid = x1;
    ep.ldr = D;
    ep.bias = atc<float>(prepared, P.b_fc2);
    if (c->variant == DIT_MMH3) {
      ep.mods = mods;
      ep.mstride = 6 * D;
      ep.goff = 5 * D;
      ep.rows = rows;
    }
    HIP_TRY(dit::gemm(dt, dit::EPI_GATED_RES, false, a, F, atc<char>(prepared, P.w_fc2), F, n, D, F, ep, s),
            "fc2 gemm");
  }
  pm.mark(8);
  return DIT_OK;
}

dit_status dit_block_forward(const dit_config* c, const void* prepared, const float* x, int32_t n,
                             const int32_t* rows, const float* pos, const double* sigmas,
                             int32_t n_sigmas, float* out, void* workspace, size_t ws_bytes,
                             void* stream) {
  return block_forward_impl(c, prepared, x, n, rows, pos, sigmas, n_sigmas, nullptr, nullptr, 0,
                            out, workspace, ws_bytes, stream);
}

dit_status dit_block_forward_packed(const dit_config* c, const void* prepared, const float* x,
                                    int32_t n, const int32_t* rows, const float* pos,
                                    const double* sigmas, int32_t n_sigmas,
                                    const int32_t* seq_starts, int32_t nseq, float* out,
                                    void* workspace, size_t ws_bytes, void* stream) {
  if (!seq_starts) return fail(DIT_EINVAL, "seq_starts is NULL");
  return block_forward_impl(c, prepared, x, n, rows, pos, sigmas, n_sigmas, nullptr, seq_starts,
                            nseq, out, workspace, ws_bytes, stream);
}

}  // extern "C"

// The output head with the velocity's sign flip folded into alpha (-1, or
// -d(sigma_a)/d(sigma_v) for a pre-multiplied audio velocity).
dit_status dit_host::final_forward_impl(const dit_config* c, const void* prepared, const float* h, int32_t n,
                              const int32_t* rows, const double* sigmas, int32_t n_sigmas, float alpha,
                              float* out, void* workspace, size_t ws_bytes, void* stream) {
  DIT_TRY(check_config(c));
  if (!head(c)) return fail(DIT_EINVAL, "dit_final_forward needs a DIT_FINAL or DIT_ZFINAL config");
  if (bad_tokens(n)) return fail(DIT_ESHAPE, "n=%d not in [0, %d]", n, kMaxTokens);
  if (!prepared) return fail(DIT_EINVAL, "prepared is NULL");
  DIT_TRY(check_sigmas(c, sigmas, n_sigmas));
  if (n == 0) return DIT_OK;
  if (!h || !out) return fail(DIT_EINVAL, "h/out is NULL");
  if (!aligned16(h) || !aligned16(out)) return fail(DIT_EALIGN, "h/out not 16-byte aligned");
  if (!workspace) return fail(DIT_EINVAL, "workspace is NULL");
  if ((uintptr_t)workspace % kAlign) return fail(DIT_EALIGN, "workspace must be 256-byte aligned");
  dit_ws_layout L = ws_layout(c, n);
  if (ws_bytes < L.total) return fail(DIT_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, L.total);
  hipStream_t s = (hipStream_t)stream;
  PrepLayout P = prep_layout(c);
  float* mods = at<float>(workspace, L.mods);
  void* xn = at<char>(workspace, L.xn);
  DIT_TRY(launch_mods(c, prepared, sigmas, mods, at<float>(workspace, L.temb), s));
  DIT_TRY(launch_prenorm(c, prepared, h, n, rows, mods, 0, xn, s));
  dit::Epi ep;
  ep.out = out;
  ep.ldc = c->F;
  ep.bias = atc<float>(prepared, P.b_fc1);
  ep.alpha = alpha;
  HIP_TRY(dit::gemm(c->dtype, dit::EPI_STORE, false, xn, c->D, atc<char>(prepared, P.w_fc1), c->D, n,
                    c->F, c->D, ep, s),
          "head gemm");
  return DIT_OK;
}
extern "C" {

dit_status dit_final_forward(const dit_config* c, const void* prepared, const float* h, int32_t n,
                             const int32_t* rows, const double* sigmas, int32_t n_sigmas, float* out,
                             void* workspace, size_t ws_bytes, void* stream) {
  // the MMH3 head predicts toward the data: the velocity is its negative
  const float alpha = c && c->variant == DIT_ZFINAL ? 1.0f : -1.0f;
  return final_forward_impl(c, prepared, h, n, rows, sigmas, n_sigmas, alpha, out, workspace, ws_bytes,
                            stream);
}

dit_status dit_linear(int32_t dtype, const void* a, int32_t lda, int32_t m, int32_t k, const void* w,
                      int32_t nout, const float* bias, float alpha, float* out, void* stream) {
  if (dtype != DIT_F32 && dtype != DIT_BF16) return fail(DIT_EDTYPE, "unknown dtype %d", dtype);
  if (m < 0 || k <= 0 || nout <= 0 || lda < k) return fail(DIT_ESHAPE, "m=%d k=%d nout=%d lda=%d", m, k, nout, lda);
  const bool bf = dtype == DIT_BF16;
  if (k % (bf ? 64 : 16) || nout % (bf ? 32 : 64))
    return fail(DIT_EUNSUPPORTED, "k=%d / nout=%d: need k %% %d == 0 and nout %% %d == 0", k, nout,
                bf ? 64 : 16, bf ? 32 : 64);
  if (lda % (bf ? 8 : 4)) return fail(DIT_EALIGN, "lda=%d must keep rows 16-byte aligned", lda);
  if (!isfinite(alpha)) return fail(DIT_EINVAL, "alpha not finite");
  if (m == 0) return DIT_OK;
  if (!a || !w || !out) return fail(DIT_EINVAL, "a/w/out is NULL");
  if (!aligned16(a) || !aligned16(w) || !aligned16(out)) return fail(DIT_EALIGN, "a/w/out not 16-byte aligned");
  dit::Epi ep;
  ep.out = out;
  ep.ldc = nout;
  ep.bias = bias;
  ep.alpha = alpha;
  HIP_TRY(dit::gemm(dtype, dit::EPI_STORE, false, a, lda, w, k, m, nout, k, ep, (hipStream_t)stream),
          "linear");
  return DIT_OK;
}

dit_status dit_patchify_video(int32_t dtype, const float* x, int32_t C, int32_t T, int32_t H,
                              int32_t W, void* rows, void* stream) {
  if (dtype != DIT_F32 && dtype != DIT_BF16) return fail(DIT_EDTYPE, "unknown dtype %d", dtype);
  if (C < 0 || T < 0 || H < 0 || W < 0 || H % 2 || W % 2)
    return fail(DIT_ESHAPE, "video [%d, %d, %d, %d]: sizes >= 0, H and W even", C, T, H, W);
  if ((size_t)C * T * H * W == 0) return DIT_OK;
  if (!x || !rows) return fail(DIT_EINVAL, "x/rows is NULL");
  HIP_TRY(dit::patchify_video(dtype, x, C, T, H, W, rows, (hipStream_t)stream), "patchify");
  return DIT_OK;
}

dit_status dit_unpatchify_video(const float* rows, int32_t C, int32_t T, int32_t H, int32_t W,
                                float* x, void* stream) {
  if (C < 0 || T < 0 || H < 0 || W < 0 || H % 2 || W % 2)
    return fail(DIT_ESHAPE, "video [%d, %d, %d, %d]: sizes >= 0, H and W even", C, T, H, W);
  if ((size_t)C * T * H * W == 0) return DIT_OK;
  if (!x || !rows) return fail(DIT_EINVAL, "x/rows is NULL");
  HIP_TRY(dit::unpatchify_video(rows, C, T, H, W, x, (hipStream_t)stream), "unpatchify");
  return DIT_OK;
}

dit_status dit_patchify_image(int32_t dtype, const float* x, int32_t C, int32_t H, int32_t W,
                              void* rows, void* stream) {
  if (dtype != DIT_F32 && dtype != DIT_BF16) return fail(DIT_EDTYPE, "unknown dtype %d", dtype);
  if (C < 0 || H < 0 || W < 0 || H % 2 || W % 2)
    return fail(DIT_ESHAPE, "image [%d, %d, %d]: sizes >= 0, H and W even", C, H, W);
  if ((size_t)C * H * W == 0) return DIT_OK;
  if (!x || !rows) return fail(DIT_EINVAL, "x/rows is NULL");
  HIP_TRY(dit::patchify_image(dtype, x, C, H, W, rows, (hipStream_t)stream), "patchify_image");
  return DIT_OK;
}

dit_status dit_unpatchify_image(const float* rows, int32_t C, int32_t H, int32_t W, float* x,
                                void* stream) {
  if (C < 0 || H < 0 || W < 0 || H % 2 || W % 2)
    return fail(DIT_ESHAPE, "image [%d, %d, %d]: sizes >= 0, H and W even", C, H, W);
  if ((size_t)C * H * W == 0) return DIT_OK;
  if (!x || !rows) return fail(DIT_EINVAL, "x/rows is NULL");
  HIP_TRY(dit::unpatchify_image(rows, C, H, W, x, (hipStream_t)stream), "unpatchify_image");
  return DIT_OK;
}

dit_status dit_pack_audio(int32_t dtype, const float* x, int32_t C, int32_t T, void* rows,
                          void* stream) {
  if (dtype != DIT_F32 && dtype != DIT_BF16) return fail(DIT_EDTYPE, "unknown dtype %d", dtype);
  if (C < 0 || T < 0) return fail(DIT_ESHAPE, "audio [%d, 2, %d]", C, T);
  if ((size_t)C * T == 0) return DIT_OK;
  if (!x || !rows) return fail(DIT_EINVAL, "x/rows is NULL");
  HIP_TRY(dit::pack_audio(dtype, x, C, T, rows, (hipStream_t)stream), "pack_audio");
  return DIT_OK;
}

dit_status dit_unpack_audio(const float* rows, int32_t C, int32_t T, float* x, void* stream) {
  if (C < 0 || T < 0) return fail(DIT_ESHAPE, "audio [%d, 2, %d]", C, T);
  if ((size_t)C * T == 0) return DIT_OK;
  if (!x || !rows) return fail(DIT_EINVAL, "x/rows is NULL");
  HIP_TRY(dit::unpack_audio(rows, C, T, x, (hipStream_t)stream), "unpack_audio");
  return DIT_OK;
}

dit_status dit_stack_forward(const dit_config* c, const void* const* prepared, int32_t n_blocks,
                             const float* x, int32_t n, const int32_t* rows, const float* pos,
                             const double* sigmas, int32_t n_sigmas, const int32_t* seq_starts,
                             int32_t nseq, float* out, void* workspace, size_t ws_bytes,
                             void* stream) {
  if (n_blocks < 1) return fail(DIT_ESHAPE, "n_blocks=%d < 1", n_blocks);
  if (!prepared) return fail(DIT_EINVAL, "prepared is NULL");
  for (int i = 0; i < n_blocks; ++i)
    if (!prepared[i]) return fail(DIT_EINVAL, "prepared[%d] is NULL", i);
  for (int i = 0; i < n_blocks; ++i)
    DIT_TRY(block_forward_impl(c, prepared[i], i == 0 ? x : out, n, rows, pos, sigmas, n_sigmas,
                               nullptr, seq_starts, nseq, out, workspace, ws_bytes, stream));
  return DIT_OK;
}

dit_status dit_block_forward_mods(const dit_config* c, const void* prepared, const float* x,
                                  int32_t n, const int32_t* rows, const float* pos,
                                  const float* mods, const int32_t* seq_starts, int32_t nseq,
                                  float* out, void* workspace, size_t ws_bytes, void* stream) {
  if (!mods) return fail(DIT_EINVAL, "mods is NULL");
  return block_forward_impl(c, prepared, x, n, rows, pos, nullptr, 0, mods, seq_starts, nseq, out,
                            workspace, ws_bytes, stream);
}

dit_status dit_rms_norm(const float* x, int32_t n, int32_t D, const float* g, float eps, float* out,
                        void* stream) {
  if (bad_tokens(n) || D <= 0 || D % 4 || D > 4096)
    return fail(DIT_ESHAPE, "n=%d D=%d (n <= %d, D %% 4 == 0, <= 4096)", n, D, kMaxTokens);
  if (!(eps >= 0.0f)) return fail(DIT_EINVAL, "eps must be >= 0");
  if (n == 0) return DIT_OK;
  if (!x || !g || !out) return fail(DIT_EINVAL, "x/g/out is NULL");
  if (!aligned16(x) || !aligned16(g) || !aligned16(out)) return fail(DIT_EALIGN, "x/g/out not 16-byte aligned");
  HIP_TRY(dit::norm_mod(dit::NORM_RMS, dit::MOD_NONE, false, x, n, D, g, nullptr, eps, nullptr, 0,
                        nullptr, 0, 0, out, (hipStream_t)stream),
          "rms_norm");
  return DIT_OK;
}

}  // extern "C"
