// C ABI of libdit.so, model level: the packed layout of an evaluation, the
// timestep-slot plan, one MMH3 denoise evaluation and the Z-Image transformer
// forward, all composed from the block-level entry points and kernels.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "../../include/dit.h"
#include "api_internal.h"
#include "dit_kernels.h"

using namespace dit_host;

extern "C" {

// ------------------------------------------------------------ MMH3 layout ----
}  // extern "C"

namespace {
// Latent frames a video token spans, cycling with period 5, rescaled onto the
// time axis ([MMH3] FRAME_PER_TOKEN, FRAME_RESCALE).
constexpr double kFrameRescale = 5.0 / 3.0;
double frame_t(int k) {
  static const double span[5] = {1.0, 4.0, 4.0, 4.0, 4.0};
  return kFrameRescale * span[k % 5];
}
// dim/2 grid points of one spatial axis spread over a window of width dim /
// sqrt(area) centred on 1/2, times 32 ([MMH3] axis_from_sqrt_area).
std::vector<double> frac_axis(int dim, double sqrt_area) {
  const double r = dim / sqrt_area;
  const int m = dim / 2;
  std::vector<double> a(m);
  for (int i = 0; i < m; ++i) a[i] = ((1.0 - r) / 2.0 + i * (r / m)) * 32.0;
  return a;
}
}  // namespace

extern "C" {

int32_t dit_mmh3_layout(int32_t text_len, int32_t latent_t, int32_t lat_h, int32_t lat_w,
                        int32_t audio_t, const int32_t* keyframes, int32_t n_keyframes,
                        const dit_layout_ref* refs, int32_t n_refs, double* pos, int32_t max_rows,
                        dit_segment* segs, int32_t max_segs, int32_t* n_segs) {
  if (text_len < 0 || latent_t < 0 || audio_t < 0 || lat_h < 2 || lat_w < 2 || n_keyframes < 0 ||
      n_refs < 0)
    return fail(DIT_ESHAPE, "layout sizes: counts >= 0, lat_h and lat_w >= 2");
  if ((n_keyframes && !keyframes) || (n_refs && !refs)) return fail(DIT_EINVAL, "keyframes/refs is NULL");
  // the rows the layout will hold, counted before it is built (int32 row indices, and
  // far below what the host buffers could take)
  const double hw = (double)(lat_h / 2) * (lat_w / 2);
  double est = text_len + 2.0 * audio_t + (double)latent_t * hw + (double)n_keyframes * hw;
  for (int r = 0; r < n_refs; ++r) {
    const dit_layout_ref& f = refs[r];
    const double rhw = (double)std::max(f.lat_h / 2, 0) * std::max(f.lat_w / 2, 0);
    if (f.kind == DIT_SEG_REF_IMAGE) est += rhw;
    else if (f.kind == DIT_SEG_VIDEO) est += 2.0 * std::max(f.audio_t, 0) + std::max(f.latent_t, 0) * rhw;
    else if (f.kind == DIT_SEG_REF_AUDIO) est += 2.0 * std::max(f.audio_t, 0);
  }
  if (est > (double)kMaxTokens)
    return fail(DIT_ESHAPE, "layout of %.0f rows exceeds %d", est, kMaxTokens);
  try {
  std::vector<double> P;  // (t, h, w) per row
  std::vector<dit_segment> G;
  auto row = [&](double t, double h, double w) { P.push_back(t); P.push_back(h); P.push_back(w); };
  auto nrows = [&]() { return (int32_t)(P.size() / 3); };
  auto seg = [&](int kind, int start) { G.push_back(dit_segment{kind, start, nrows()}); };
  auto stereo = [&](double c0, int t, double w_lo, double w_hi) {
    for (int ch = 0; ch < 2; ++ch)
      for (int i = 0; i < t; ++i) row(c0 + i, 0.0, ch ? w_hi : w_lo);
  };
  const double sq = sqrt((double)lat_h * lat_w);
  const std::vector<double> ha = frac_axis(lat_h, sq), wa = frac_axis(lat_w, sq);
  for (int i = 0; i < text_len; ++i) row(i, 0.0, 0.0);
  seg(DIT_SEG_TEXT, 0);
  double cursor = text_len;
  for (int r = 0; r < n_refs; ++r) {
    const dit_layout_ref& f = refs[r];
    const int start = nrows();
    if (f.kind == DIT_SEG_REF_IMAGE || f.kind == DIT_SEG_VIDEO) {
      if (f.lat_h < 2 || f.lat_w < 2 || f.latent_t < 0 || f.audio_t < 0)
        return fail(DIT_ESHAPE, "reference %d: lat_h, lat_w >= 2", r);
      const double rs = sqrt((double)f.lat_h * f.lat_w);
      const std::vector<double> rh = frac_axis(f.lat_h, rs), rw = frac_axis(f.lat_w, rs);
      if (f.kind == DIT_SEG_REF_IMAGE) {
        for (double h : rh)
          for (double w : rw) row(cursor, h, w);
        seg(DIT_SEG_REF_IMAGE, start);
        cursor += 1.0;
      } else {  // a clip: its soundtrack first, then its frames, from the same origin
        if (f.audio_t > 0) {
          stereo(cursor, f.audio_t, rw.front(), rw.back());
          seg(DIT_SEG_REF_AUDIO, start);
        }
        const int fs = nrows();
        double t = cursor, spans = 0.0;
        for (int k = 0; k < f.latent_t; ++k) {
          for (double h : rh)
            for (double w : rw) row(t, h, w);
          t += frame_t(k);
          spans += frame_t(k);
        }
        seg(DIT_SEG_REF_IMAGE, fs);
        cursor += std::max((double)f.audio_t, spans);
      }
    } else if (f.kind == DIT_SEG_REF_AUDIO) {
      if (f.audio_t < 0) return fail(DIT_ESHAPE, "reference %d: audio_t < 0", r);
      if (f.audio_t > 0) {
        stereo(cursor, f.audio_t, wa.front(), wa.back());
        seg(DIT_SEG_REF_AUDIO, start);
      }
      cursor += f.audio_t;
    } else {
      return fail(DIT_EINVAL, "reference %d: unknown kind %d", r, f.kind);
    }
  }
  double spans = 0.0;
  for (int k = 0; k < latent_t; ++k) spans += frame_t(k);
  for (int i = 0; i < n_keyframes; ++i) {
    const int pix = keyframes[2 * i], count = keyframes[2 * i + 1];
    double t;
    if (pix == 0) t = cursor;
    else if (count > 0 && pix == count - 1) t = cursor + spans - kFrameRescale;
    else return fail(DIT_EINVAL, "keyframe %d: pixel index %d is neither the first nor the last of %d", i, pix, count);
    const int start = nrows();
    for (double h : ha)
      for (double w : wa) row(t, h, w);
    seg(DIT_SEG_COND, start);
  }
  int start = nrows();
  stereo(cursor, audio_t, wa.front(), wa.back());
  seg(DIT_SEG_AUDIO, start);
  start = nrows();
  double t = cursor;
  for (int k = 0; k < latent_t; ++k) {
    for (double h : ha)
      for (double w : wa) row(t, h, w);
    t += frame_t(k);
  }
  seg(DIT_SEG_VIDEO, start);
  if (n_segs) *n_segs = (int32_t)G.size();
  if (pos) {
    if (max_rows < nrows() || max_segs < (int32_t)G.size() || !segs)
      return fail(DIT_ESHAPE, "layout needs %d rows and %zu segments (have %d, %d)", nrows(), G.size(), max_rows, max_segs);
    memcpy(pos, P.data(), P.size() * sizeof(double));
    memcpy(segs, G.data(), G.size() * sizeof(dit_segment));
  }
  g_err[0] = 0;
  return nrows();
  } DIT_CATCH_ALL
}

int32_t dit_mmh3_slots(double sigma_v, double shift_video, double shift_audio, double cond_aug,
                       double cond_aug_audio, int32_t has_cond, int32_t has_ref_audio,
                       double slot_sigmas[4], int32_t slot_of[4]) {
  if (!slot_sigmas || !slot_of) return fail(DIT_EINVAL, "slot_sigmas/slot_of is NULL");
  if (!isfinite(sigma_v) || !isfinite(shift_video) || !isfinite(shift_audio) || !isfinite(cond_aug) ||
      !isfinite(cond_aug_audio))
    return fail(DIT_EINVAL, "non-finite slot input");
  if (!(shift_video > 0.0) || !(shift_audio > 0.0)) return fail(DIT_EINVAL, "flow shifts must be > 0");
  const double sv = std::max(sigma_v, 1e-6);
  const double tv = 1.0 - sv;
  const double ta = 1.0 - dit_sigma_remap(sv, shift_video, shift_audio);
  if (!isfinite(ta)) return fail(DIT_EINVAL, "audio sigma of sigma_v=%g is not finite", sigma_v);
  double t[4] = {tv, ta, 0.0, 0.0};
  int nt = 2;
  const double tc = std::max(tv, cond_aug), tca = std::max(ta, cond_aug_audio);
  if (has_cond) t[nt++] = tc;
  if (has_ref_audio) t[nt++] = tca;
  std::sort(t, t + nt);
  nt = (int)(std::unique(t, t + nt) - t);
  auto slot = [&](double v) { return (int32_t)(std::find(t, t + nt, v) - t); };
  for (int i = 0; i < 4; ++i) slot_sigmas[i] = i < nt ? 1.0 - t[i] : 0.0;
  slot_of[0] = slot(tv);
  slot_of[1] = slot(ta);
  slot_of[2] = has_cond ? slot(tc) : -1;
  slot_of[3] = has_ref_audio ? slot(tca) : -1;
  return nt;
}

// ------------------------------------------------------------ MMH3 model ----
}  // extern "C"

namespace {
struct ModelPlan {
  int n = 0, nv = 0, na = 0, text = -1, video = -1, audio = -1, ncond = 0;
  // workspace offsets
  size_t h = 0, rows = 0, hrows = 0, prow = 0, hout = 0, bws = 0, hws = 0, total = 0;
};

dit_status plan_model(const dit_mmh3_model* m, const dit_segment* segs, int32_t nseg, ModelPlan* P) {
  if (!m || !segs || nseg < 1) return fail(DIT_EINVAL, "model/segments missing");
  if (!m->block || !m->head_video || !m->blocks || m->n_blocks < 1)
    return fail(DIT_EINVAL, "model needs a block config, blocks and a video head");
  DIT_TRY(check_config(m->block));
  if (m->block->variant != DIT_MMH3) return fail(DIT_EINVAL, "model blocks must be DIT_MMH3");
  // token rows are slot * 3 + tag over the page's three modalities (video 0,
  // text 1, audio 2); the modulation table's row stride is the block's tags
  if (m->block->tags != 3)
    return fail(DIT_EUNSUPPORTED, "the evaluation's blocks need tags = 3 (video, text, audio), got %d",
                m->block->tags);
  if (m->audio_slope_rescale != 0 && m->audio_slope_rescale != 1)
    return fail(DIT_EINVAL, "audio_slope_rescale=%d (0 or 1)", m->audio_slope_rescale);
  DIT_TRY(check_config(m->head_video));
  if (m->head_video->variant != DIT_FINAL || m->head_video->F != 4 * m->latent_c ||
      m->head_video->D != m->block->D || m->head_video->slots != m->block->slots)
    return fail(DIT_EINVAL, "video head: DIT_FINAL, F = 4 * latent_c, the blocks' D and slots");
  const bool bf = m->block->dtype == DIT_BF16;
  if (m->latent_c > 65536 || m->audio_c > 65536) return fail(DIT_EUNSUPPORTED, "latent_c/audio_c > 65536");
  if (m->latent_c <= 0 || (4 * m->latent_c) % (bf ? 64 : 16))
    return fail(DIT_EUNSUPPORTED, "latent_c=%d: 4 * latent_c must be a multiple of %d", m->latent_c, bf ? 64 : 16);
  int pos = 0;
  for (int i = 0; i < nseg; ++i) {
    const dit_segment& g = segs[i];
    if (g.start != pos || g.stop < g.start) return fail(DIT_ESHAPE, "segment %d [%d, %d) must start at %d", i, g.start, g.stop, pos);
    pos = g.stop;
    switch (g.kind) {
      case DIT_SEG_TEXT: if (P->text >= 0) return fail(DIT_EINVAL, "two TEXT segments"); P->text = i; break;
      case DIT_SEG_VIDEO: if (P->video >= 0) return fail(DIT_EINVAL, "two VIDEO segments"); P->video = i; break;
      case DIT_SEG_AUDIO: if (P->audio >= 0) return fail(DIT_EINVAL, "two AUDIO segments"); P->audio = i; break;
      case DIT_SEG_COND: P->ncond++; break;
      default: return fail(DIT_EINVAL, "segment %d: unknown kind %d", i, g.kind);
    }
  }
  if (P->video < 0) return fail(DIT_EINVAL, "no VIDEO segment");
  if (bad_tokens(pos)) return fail(DIT_ESHAPE, "%d tokens (at most %d)", pos, kMaxTokens);
  P->n = pos;
  P->nv = segs[P->video].stop - segs[P->video].start;
  P->na = P->audio >= 0 ? segs[P->audio].stop - segs[P->audio].start : 0;
  if (P->audio >= 0) {
    if (!m->head_audio || !m->audio_patch_w) return fail(DIT_EINVAL, "an AUDIO segment needs the audio head and patch");
    DIT_TRY(check_config(m->head_audio));
    if (m->head_audio->variant != DIT_FINAL || m->head_audio->F != m->audio_c ||
        m->head_audio->D != m->block->D || m->head_audio->slots != m->block->slots)
      return fail(DIT_EINVAL, "audio head: DIT_FINAL, F = audio_c, the blocks' D and slots");
    if (m->audio_c <= 0 || m->audio_c % (bf ? 64 : 16))
      return fail(DIT_EUNSUPPORTED, "audio_c=%d must be a multiple of %d", m->audio_c, bf ? 64 : 16);
  }
  const size_t D = m->block->D, es = bf ? 2 : 4;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  int max_cond_rows = 0;
  for (int i = 0; i < nseg; ++i)
    if (segs[i].kind == DIT_SEG_COND) max_cond_rows = std::max(max_cond_rows, segs[i].stop - segs[i].start);
  const size_t prow_elems = std::max({(size_t)P->nv * 4 * m->latent_c, (size_t)max_cond_rows * 4 * m->latent_c,
                                      (size_t)P->na * std::max(m->audio_c, 1)});
  const size_t hout_elems = std::max((size_t)P->nv * 4 * m->latent_c, (size_t)P->na * std::max(m->audio_c, 1));
  P->h = take((size_t)P->n * D * 4);
  P->rows = take((size_t)P->n * 4);
  P->hrows = take((size_t)std::max(P->nv, P->na) * 4);
  P->prow = take(prow_elems * es);
  P->hout = take(hout_elems * 4);
  P->bws = take(ws_layout(m->block, P->n).total);
  size_t hws = ws_layout(m->head_video, P->nv).total;
  if (P->audio >= 0) hws = std::max(hws, ws_layout(m->head_audio, P->na).total);
  P->hws = take(hws);
  P->total = off;
  return DIT_OK;
}
}  // namespace

extern "C" {

size_t dit_mmh3_workspace_size(const dit_mmh3_model* m, const dit_segment* segs, int32_t nseg) {
  ModelPlan P;
  return plan_model(m, segs, nseg, &P) == DIT_OK ? P.total : 0;
}

dit_status dit_mmh3_forward(const dit_mmh3_model* m, const dit_segment* segs, int32_t nseg,
                            const float* pos, const float* text, const int32_t* text_tags,
                            const float* video, int32_t T,
                            int32_t H, int32_t W, const float* audio, int32_t Ta,
                            const float* const* cond, double sigma_v, float* video_out,
                            float* audio_out, void* workspace, size_t ws_bytes, void* stream) {
  ModelPlan P;
  DIT_TRY(plan_model(m, segs, nseg, &P));
  const dit_config* bc = m->block;
  const int D = bc->D, C = m->latent_c;
  if (T <= 0 || H <= 0 || W <= 0 || H % 2 || W % 2 || (long long)P.nv != (long long)T * (H / 2) * (W / 2))
    return fail(DIT_ESHAPE, "video [%d, %d, %d, %d] does not give the VIDEO segment's %d rows", C, T, H, W, P.nv);
  if (P.audio >= 0 && P.na != 2 * Ta) return fail(DIT_ESHAPE, "audio length %d does not give %d rows", Ta, P.na);
  for (int i = 0; i < nseg; ++i)
    if (segs[i].kind == DIT_SEG_COND && (long long)segs[i].stop - segs[i].start != (long long)(H / 2) * (W / 2))
      return fail(DIT_ESHAPE, "COND segment %d must hold one frame of (H/2)(W/2) rows", i);
  if (!pos || !video || !video_out || (P.audio >= 0 && (!audio || !audio_out)) ||
      (P.text >= 0 && segs[P.text].stop > segs[P.text].start && !text) || (P.ncond && !cond))
    return fail(DIT_EINVAL, "an input or output pointer is NULL");
  if (!isfinite(sigma_v)) return fail(DIT_EINVAL, "sigma_v not finite");
  for (int k = 0; k < P.ncond; ++k)
    if (!cond[k]) return fail(DIT_EINVAL, "condition frame %d is NULL", k);
  if (!workspace || (uintptr_t)workspace % kAlign) return fail(DIT_EALIGN, "workspace NULL or not 256-byte aligned");
  if (ws_bytes < P.total) return fail(DIT_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, P.total);
  hipStream_t s = (hipStream_t)stream;

  // timestep slots and per-token rows ([MMH3] MiniMaxH3::forward)
  double ssig[4];
  int32_t slot[4];
  const int nt = dit_mmh3_slots(sigma_v, m->shift_video, m->shift_audio, m->cond_aug, m->cond_aug_audio,
                                P.ncond > 0, 0, ssig, slot);
  if (nt < 0) return (dit_status)nt;
  if (nt > bc->slots) return fail(DIT_EUNSUPPORTED, "the evaluation needs %d slots, the blocks have %d", nt, bc->slots);
  double sig[kMaxSlots];  // slots beyond the plan: unused rows
  for (int i = 0; i < bc->slots; ++i) sig[i] = i < nt ? ssig[i] : ssig[nt - 1];
  float* h = at<float>(workspace, P.h);
  int* rows = at<int>(workspace, P.rows);
  int* hrows = at<int>(workspace, P.hrows);
  void* prow = at<char>(workspace, P.prow);
  float* hout = at<float>(workspace, P.hout);
  const int dt = bc->dtype;
  int ci = 0;
  for (int i = 0; i < nseg; ++i) {
    const dit_segment& g = segs[i];
    const int len = g.stop - g.start;
    if (len == 0) continue;
    int row = 0;
    switch (g.kind) {  // slot * 3 + tag (video 0, text 1, audio 2)
      case DIT_SEG_TEXT: row = slot[0] * 3 + 1; break;
      case DIT_SEG_VIDEO: row = slot[0] * 3 + 0; break;
      case DIT_SEG_AUDIO: row = slot[1] * 3 + 2; break;
      default: row = slot[2] * 3 + 0; break;
    }
    if (g.kind == DIT_SEG_TEXT && text_tags)  // per-token modality of the prompt span
      HIP_TRY(dit::rows_from_tags(text_tags, len, slot[0] * 3, rows + g.start, s), "token rows");
    else
      HIP_TRY(dit::fill_i32(rows + g.start, len, row, s), "token rows");
    float* hs = h + (size_t)g.start * D;
    if (g.kind == DIT_SEG_TEXT) {
      HIP_TRY(hipMemcpyAsync(hs, text, (size_t)len * D * 4, hipMemcpyDeviceToDevice, s), "text rows");
    } else if (g.kind == DIT_SEG_VIDEO || g.kind == DIT_SEG_COND) {
      const float* src = g.kind == DIT_SEG_VIDEO ? video : cond[ci++];
      HIP_TRY(dit::patchify_video(dt, src, C, g.kind == DIT_SEG_VIDEO ? T : 1, H, W, prow, s), "patchify");
      DIT_TRY(dit_linear(dt, prow, 4 * C, len, 4 * C, m->video_patch_w, D, m->video_patch_b, 1.0f, hs, s));
    } else {
      HIP_TRY(dit::pack_audio(dt, audio, m->audio_c, Ta, prow, s), "pack_audio");
      DIT_TRY(dit_linear(dt, prow, m->audio_c, len, m->audio_c, m->audio_patch_w, D, m->audio_patch_b, 1.0f, hs, s));
    }
  }
  // blocks, in place on h
  DIT_TRY(dit_stack_forward(bc, m->blocks, m->n_blocks, h, P.n, rows, pos, sig, bc->slots, nullptr, 0, h,
                            at<char>(workspace, P.bws), ws_layout(bc, P.n).total, s));
  // heads: the row of a head is the stream's timestep slot
  const size_t hws = P.total - P.hws;
  {
    const dit_segment& g = segs[P.video];
    HIP_TRY(dit::fill_i32(hrows, P.nv, slot[0], s), "head rows");
    DIT_TRY(dit_final_forward(m->head_video, m->head_video_w, h + (size_t)g.start * D, P.nv, hrows, sig,
                              bc->slots, hout, at<char>(workspace, P.hws), hws, s));
    HIP_TRY(dit::unpatchify_video(hout, C, T, H, W, video_out, s), "unpatchify");
  }
  if (P.audio >= 0 && P.na > 0) {
    const dit_segment& g = segs[P.audio];
    HIP_TRY(dit::fill_i32(hrows, P.na, slot[1], s), "head rows");
    const double slope =
        m->audio_slope_rescale ? dit_sigma_remap_slope(sigma_v, m->shift_video, m->shift_audio) : 1.0;
    DIT_TRY(final_forward_impl(m->head_audio, m->head_audio_w, h + (size_t)g.start * D, P.na, hrows, sig,
                               bc->slots, (float)-slope, hout, at<char>(workspace, P.hws), hws, s));
    HIP_TRY(dit::unpack_audio(hout, m->audio_c, Ta, audio_out, s), "unpack_audio");
  }
  return DIT_OK;
}

// ------------------------------------------------------------ Z-Image model ----
}  // extern "C"

namespace {
struct ZPlan {
  int ni = 0, nc = 0, n = 0;
  size_t h = 0, prow = 0, crow = 0, hout = 0, bws = 0, bws_bytes = 0, total = 0;
};

// Runs blocks [b0, b1) of a stack in place on h (nothing when the range is empty).
dit_status run_blocks(const dit_config* c, const void* const* prep, int b0, int b1, float* h, int n,
                      const float* pos, const double* sig, int nsig, void* ws, size_t wsb, hipStream_t s) {
  if (b1 <= b0 || n == 0) return DIT_OK;
  return dit_stack_forward(c, prep + b0, b1 - b0, h, n, nullptr, pos, sig, nsig, nullptr, 0, h, ws, wsb, s);
}

dit_status plan_zimage(const dit_zimage_model* m, int H, int W, int cap_len, ZPlan* P) {
  if (!m) return fail(DIT_EINVAL, "model is NULL");
  if (!m->block || !m->final_layer || !m->final_w || (m->n_context_refiners > 0 && !m->context))
    return fail(DIT_EINVAL, "model needs block and final-layer configs, final weights and (with context "
                            "refiners) their config");
  DIT_TRY(check_config(m->block));
  if (m->context) DIT_TRY(check_config(m->context));
  DIT_TRY(check_config(m->final_layer));
  const dit_config *b = m->block, *c = m->context, *f = m->final_layer;
  if (b->variant != DIT_ZIMAGE || (c && c->variant != DIT_ZCONTEXT) || f->variant != DIT_ZFINAL)
    return fail(DIT_EINVAL, "configs must be DIT_ZIMAGE, DIT_ZCONTEXT and DIT_ZFINAL");
  if ((c && (c->D != b->D || c->H != b->H || c->hd != b->hd || c->dtype != b->dtype)) || f->D != b->D ||
      f->dtype != b->dtype)
    return fail(DIT_EINVAL, "block, context refiner and final layer must share D, heads and dtype");
  if (m->in_channels > 65536) return fail(DIT_EUNSUPPORTED, "in_channels=%d > 65536", m->in_channels);
  if (f->F != 4 * m->in_channels) return fail(DIT_EINVAL, "final layer F=%d != 4 * in_channels", f->F);
  if (m->n_layers < 0 || m->n_noise_refiners < 0 || m->n_context_refiners < 0)
    return fail(DIT_EINVAL, "negative block counts");
  if ((m->n_layers && !m->layers) || (m->n_noise_refiners && !m->noise_refiners) ||
      (m->n_context_refiners && !m->context_refiners))
    return fail(DIT_EINVAL, "block arrays are NULL");
  if (!m->x_embed_w || !m->cap_embed_w || !m->cap_norm) return fail(DIT_EINVAL, "embedder weights are NULL");
  const bool bf = b->dtype == DIT_BF16;
  const int km = bf ? 64 : 16;
  if (m->in_channels <= 0 || (4 * m->in_channels) % km)
    return fail(DIT_EUNSUPPORTED, "4 * in_channels=%d must be a multiple of %d", 4 * m->in_channels, km);
  if (m->cap_dim <= 0 || m->cap_dim % km || m->cap_dim > 4096)
    return fail(DIT_EUNSUPPORTED, "cap_dim=%d must be a multiple of %d and <= 4096", m->cap_dim, km);
  if (!(m->cap_eps >= 0.0f)) return fail(DIT_EINVAL, "cap_eps must be >= 0");
  if (H <= 0 || W <= 0 || H % 2 || W % 2 || cap_len < 0 ||
      bad_tokens((long long)(H / 2) * (W / 2) + cap_len))
    return fail(DIT_ESHAPE, "image %d x %d (even, > 0), caption %d: at most %d tokens", H, W, cap_len,
                kMaxTokens);
  P->ni = (H / 2) * (W / 2);
  P->nc = cap_len;
  P->n = P->ni + P->nc;
  const size_t D = b->D, es = bf ? 2 : 4;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  P->h = take((size_t)P->n * D * 4);
  P->prow = take((size_t)P->ni * 4 * m->in_channels * es);
  P->crow = take((size_t)std::max(P->nc, 1) * m->cap_dim * es);
  P->hout = take((size_t)P->ni * 4 * m->in_channels * 4);
  P->bws_bytes = std::max({ws_layout(b, P->n).total, c ? ws_layout(c, std::max(P->nc, 1)).total : (size_t)0,
                           ws_layout(f, P->ni).total});
  P->bws = take(P->bws_bytes);
  P->total = off;
  return DIT_OK;
}
}  // namespace

extern "C" {

size_t dit_zimage_workspace_size(const dit_zimage_model* m, int32_t H, int32_t W, int32_t cap_len) {
  ZPlan P;
  return plan_zimage(m, H, W, cap_len, &P) == DIT_OK ? P.total : 0;
}

dit_status dit_zimage_forward(const dit_zimage_model* m, const float* latents, int32_t H, int32_t W,
                              const float* cap_feats, int32_t cap_len, const float* pos, double t,
                              int32_t step, dit_zimage_cache* cache, float* out, void* workspace,
                              size_t ws_bytes, void* stream) {
  ZPlan P;
  DIT_TRY(plan_zimage(m, H, W, cap_len, &P));
  if (!latents || !pos || !out || (cap_len > 0 && !cap_feats)) return fail(DIT_EINVAL, "input/output is NULL");
  if (!aligned16(latents) || !aligned16(pos) || !aligned16(out) || (cap_feats && !aligned16(cap_feats)))
    return fail(DIT_EALIGN, "inputs/outputs not 16-byte aligned");
  if (!isfinite(t)) return fail(DIT_EINVAL, "t is not finite");
  if (!workspace) return fail(DIT_EINVAL, "workspace is NULL");
  if ((uintptr_t)workspace % kAlign) return fail(DIT_EALIGN, "workspace must be 256-byte aligned");
  if (ws_bytes < P.total) return fail(DIT_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, P.total);
  if (cache) {
    if (cache->interval < 1) return fail(DIT_EINVAL, "cache interval=%d < 1", cache->interval);
    if (cache->layers < 0 || cache->layers > m->n_layers)
      return fail(DIT_EINVAL, "cache layers=%d outside [0, %d]", cache->layers, m->n_layers);
    if (cache->layers > 0 && !cache->shallow) return fail(DIT_EINVAL, "cache->shallow is NULL");
    if (cap_len > 0 && !cache->caption) return fail(DIT_EINVAL, "cache->caption is NULL");
    if (step < 0) return fail(DIT_EINVAL, "step=%d < 0", step);
  }
  hipStream_t s = (hipStream_t)stream;
  const dit_config* b = m->block;
  const int D = b->D, C = m->in_channels, dt = b->dtype;
  const size_t rowb = (size_t)D * 4;
  float* h = at<float>(workspace, P.h);
  float* hc = h + (size_t)P.ni * D;  // caption rows of the unified stream
  const float* pos_c = pos + (size_t)P.ni * 3;
  void* bws = at<char>(workspace, P.bws);
  const double sig[1] = {t};
  // [ZIMG] ForwardWithCache: on a step that is not a refresh, every shallow layer reads its
  // stored output, so the stream after them is the stored one and the image embedding and
  // noise refiners before them have no effect on the result.
  const int nshallow = cache ? cache->layers : 0;
  const bool refresh = cache ? step % cache->interval == 0 : true;
  const bool reuse = cache && nshallow > 0 && !refresh && cache->shallow_valid;
  if (reuse) {
    HIP_TRY(hipMemcpyAsync(h, cache->shallow, (size_t)P.n * rowb, hipMemcpyDeviceToDevice, s), "reuse layers");
  } else {
    // image: patchify + x embedder, then the noise refiners (modulated, image tokens only)
    HIP_TRY(dit::patchify_image(dt, latents, C, H, W, at<char>(workspace, P.prow), s), "patchify_image");
    DIT_TRY(dit_linear(dt, at<char>(workspace, P.prow), 4 * C, P.ni, 4 * C, m->x_embed_w, D, m->x_embed_b, 1.0f,
                       h, s));
    DIT_TRY(run_blocks(b, m->noise_refiners, 0, m->n_noise_refiners, h, P.ni, pos, sig, 1, bws, P.bws_bytes, s));
    // caption: RMSNorm + cap embedder, then the context refiners; once per generation with a cache
    if (P.nc > 0) {
      if (cache && cache->caption_valid) {
        HIP_TRY(hipMemcpyAsync(hc, cache->caption, (size_t)P.nc * rowb, hipMemcpyDeviceToDevice, s), "caption");
      } else {
        HIP_TRY(dit::norm_mod(dit::NORM_RMS, dit::MOD_NONE, dt == DIT_BF16, cap_feats, P.nc, m->cap_dim, m->cap_norm,
                              nullptr, m->cap_eps, nullptr, 0, nullptr, 0, 0, at<char>(workspace, P.crow), s),
                "caption norm");
        DIT_TRY(dit_linear(dt, at<char>(workspace, P.crow), m->cap_dim, P.nc, m->cap_dim, m->cap_embed_w, D,
                           m->cap_embed_b, 1.0f, hc, s));
        DIT_TRY(run_blocks(m->context, m->context_refiners, 0, m->n_context_refiners, hc, P.nc, pos_c, nullptr, 0,
                           bws, P.bws_bytes, s));
        if (cache) {
          HIP_TRY(hipMemcpyAsync(cache->caption, hc, (size_t)P.nc * rowb, hipMemcpyDeviceToDevice, s), "store caption");
          cache->caption_valid = 1;
        }
      }
    }
    // the shallow main layers, stored on refresh steps
    DIT_TRY(run_blocks(b, m->layers, 0, nshallow, h, P.n, pos, sig, 1, bws, P.bws_bytes, s));
    if (cache && nshallow > 0 && refresh) {
      HIP_TRY(hipMemcpyAsync(cache->shallow, h, (size_t)P.n * rowb, hipMemcpyDeviceToDevice, s), "store layers");
      cache->shallow_valid = 1;
    }
  }
  DIT_TRY(run_blocks(b, m->layers, nshallow, m->n_layers, h, P.n, pos, sig, 1, bws, P.bws_bytes, s));
  // final layer on the image tokens, then back to [C, H, W]
  float* hout = at<float>(workspace, P.hout);
  DIT_TRY(final_forward_impl(m->final_layer, m->final_w, h, P.ni, nullptr, sig, 1, 1.0f, hout, bws,
                             P.bws_bytes, s));
  HIP_TRY(dit::unpatchify_image(hout, C, H, W, out, s), "unpatchify_image");
  return DIT_OK;
}

}  // extern "C"
