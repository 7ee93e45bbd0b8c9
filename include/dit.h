/*
 * dit.h - C ABI of the packed diffusion-transformer block library (libdit.so)
 * for AMD Instinct MI355X (gfx950).
 *
 * One call runs the forward pass of one DiT block over a packed token
 * sequence: text, audio and video (or image) tokens share one sequence and are
 * told apart only by a per-token modulation row.  Citation tags:
 *
 *   [MMH3]   docs.rs source page of cortiq-engine 0.5.72, src/mmh3.rs
 *   [SIGLIP] docs.rs source page of ffai-argus 0.7.0, src/siglip.rs
 *   [ZIMG]   ollama fork, x/imagegen/models/zimage/transformer.go
 *   [ENC]    docs.rs source page of inferencelayer 0.2.1, src/encoder_cpu.rs
 *
 * Conventions for every entry point:
 *   - Data pointers are DEVICE memory owned by the caller, except where an
 *     argument is marked "host".  The library never allocates or frees device
 *     memory: prepared weights and the workspace are caller buffers sized by
 *     the *_size queries.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     asynchronously; nothing synchronizes inside the library.
 *   - All arguments are validated on the host before anything is launched.
 *     On failure nothing is written and a negative dit_status is returned; the
 *     message is in dit_last_error() (thread-local).  Launch failures return
 *     DIT_EHIP.  Device faults surface at the caller's next synchronization.
 *   - n == 0 is valid and does nothing.  Every token count (a block's n, an
 *     evaluation's segments, a Z-Image image plus caption, a layout) is at
 *     most 2^24; larger ones are refused with DIT_ESHAPE (size queries: 0).
 *   - There is no CPU fallback: every step runs in the library's HIP kernels.
 *   - HIP graph capture: every launch goes to `stream`, nothing allocates and
 *     padding is cleared by kernels (no memset nodes), so calls can be
 *     captured.  Host arguments are frozen into the captured launches: the
 *     sigmas (as slot coordinates), seq_starts, n and the launch plans.  A
 *     replay of a captured dit_block_forward therefore uses the capture-time
 *     timestep.  For a new timestep per replay, capture
 *     dit_block_forward_mods (its modulation rows are read from device
 *     memory) and refresh those rows with dit_adaln_eval, outside the graph,
 *     before each replay.
 *   - Supported shapes: hd in {64, 128}, D = H*hd, D % 128 == 0,
 *     F % 128 == 0, D <= 4096, 1 <= slots <= 8, rank <= 64, grid >= 2;
 *     pointers 16-byte aligned; tensors contiguous row-major.
 */
#ifndef DIT_H
#define DIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DIT_OK = 0,
  DIT_EINVAL = -1,       /* NULL pointer where one is required, bad value   */
  DIT_ESHAPE = -2,       /* inconsistent sizes                              */
  DIT_EDTYPE = -3,       /* unknown dtype                                   */
  DIT_EALIGN = -4,       /* pointer not 16-byte aligned                     */
  DIT_EWORKSPACE = -5,   /* workspace or prepared buffer too small          */
  DIT_EUNSUPPORTED = -6, /* shape outside the supported set                 */
  DIT_EHIP = -7          /* a HIP launch failed                             */
} dit_status;

/* Block variant. */
enum {
  DIT_MMH3 = 0,   /* six-chunk adaLN (shift/scale/gate x2) from a rank-r timestep-curve
                     basis, RMSNorm, qk-RMSNorm + 3-axis RoPE, SwiGLU ([MMH3] block_forward) */
  DIT_SIGLIP = 1, /* pre-LayerNorm encoder layer with biases, GELU-tanh, no modulation and
                     no RoPE; softmax scale folded into W_q, b_q ([SIGLIP] Layer::forward)    */
  DIT_ZIMAGE = 2, /* four-chunk adaLN from a sinusoidal timestep MLP, tanh gates, sandwich
                     RMSNorms, interleaved RoPE, SwiGLU ([ZIMG] TransformerBlock.Forward)     */
  DIT_REFINER = 3, /* the MMH3 block without modulation, as its token refiner runs it
                     ([MMH3] refine_text: block_forward with no mods): RMSNorm pre-norms,
                     qk-RMSNorm, plain residuals, SwiGLU; RoPE as configured (the
                     refiner itself is unrotated: rope = NONE); no sigmas          */
  DIT_FINAL = 4,   /* the MMH3 output head, not a block: RMSNorm, a single-modality
                     adaLN of two chunks (shift, scale) per timestep slot, a linear
                     head and the sign flip (tags = 1, F = output width; run by
                     dit_final_forward) ([MMH3] MiniMaxH3::forward, heads)        */
  DIT_ZCONTEXT = 5, /* the Z-Image block without modulation, as its context (caption)
                     refiner runs it ([ZIMG] TransformerBlock.Forward with no adaLN):
                     x1 = x + RMSNorm(Attn(RMSNorm(x)); post_attn_norm), out = x1 +
                     RMSNorm(FFN(RMSNorm(x1)); post_ffn_norm); no sigmas          */
  DIT_ZFINAL = 6   /* the Z-Image final layer, not a block ([ZIMG] FinalLayer.Forward):
                     temb from the timestep MLP, scale = ada_w silu(temb) + ada_b,
                     out = W (LayerNorm_noaffine(h; eps) * (1 + scale)) + b (F = output
                     width; run by dit_final_forward; no sign flip)               */
};

/* Arithmetic type of GEMM operands, attention inputs and the intermediates
 * (the residual stream x, x1 and out are always fp32). */
enum { DIT_F32 = 0, DIT_BF16 = 1 };

/* RoPE pair layout. */
enum {
  DIT_ROPE_NONE = 0,
  DIT_ROPE_SPLIT_HALF = 1,  /* pair (j, j + hd/2) ([MMH3] norm_rope_w)  */
  DIT_ROPE_INTERLEAVED = 2, /* pair (2j, 2j + 1) ([ZIMG] applyRoPE3D)  */
  DIT_ROPE_PARTIAL = 3      /* the checkpoint form of [MMH3] rope_angles / norm_rope_w: k =
                               rope_axes[0]/2 frequencies (weights.rope_freq) shared by the
                               three axes (rope_axes all equal, 3 * rope_axes[0] <= hd), P = 3k
                               angles per token, angle j = pos[j / k] * rope_freq[j % k], pair
                               (j, j + P) for j < P, head dims [2P, hd) not rotated; rope_theta
                               unused.  DIT_MMH3 and DIT_REFINER only. */
};

typedef struct dit_config {
  int32_t variant;       /* DIT_MMH3 / DIT_SIGLIP / DIT_ZIMAGE / DIT_REFINER / DIT_FINAL */
  int32_t dtype;         /* DIT_F32 / DIT_BF16                                          */
  int32_t D, H, hd, F;   /* hidden, heads, head dim (D = H*hd), FFN hidden (FINAL: output
                            width, a multiple of 32 for bf16 and of 64 for fp32)         */
  int32_t slots;         /* MMH3: timestep slots S                                      */
  int32_t tags;          /* MMH3: modality tags T (3: video 0, text 1, audio 2)         */
  int32_t rank;          /* MMH3: adaLN curve rank r (24)                               */
  int32_t grid;          /* MMH3: adaLN table rows G (1025)                             */
  int32_t rope;          /* DIT_ROPE_*                                                  */
  int32_t rope_axes[3];  /* dims per position axis (t, h, w); sum = hd                  */
  double rope_theta;     /* frequency base: axis a, pair m turns by pos * theta^(-2m/d_a) */
  float eps;             /* block norm epsilon (RMSNorm or LayerNorm)                   */
  float qk_eps;          /* qk-RMSNorm epsilon                                          */
  int32_t temb_freq;     /* ZIMAGE: sinusoid width (256)                                */
  int32_t temb_hidden;   /* ZIMAGE: timestep MLP hidden width (1024)                    */
  float t_scale;         /* ZIMAGE: timestep multiplier before the sinusoid (1000)      */
  int32_t adaln_shared;  /* MMH3 / FINAL: 0 = slot-major basis (one block of rows per slot);
                            1 = one slot's rows [T*E*D, r] (and bias [T*E*D]) evaluated at
                            every slot's timestep, as [MMH3] Adaln::eval applies one W at
                            each distinct timestep                                      */
} dit_config;

/* Raw weights, device pointers.  GEMM weights (w_*) are [out, in] row-major in
 * the config's dtype (float or bfloat16); everything else is fp32.  Pointers a
 * variant does not use may be NULL.
 *   MMH3:   norm1, norm2 [D]; w_qkv [3D, D] (rows q | k | v); w_out [D, D];
 *           q_norm, k_norm [hd]; w_fc1 [2F, D] (rows gate | up); w_fc2 [D, F];
 *           adaln_basis [S*T*6*D, r] (slot-major: rows of slot s are
 *           [s*T*6*D, (s+1)*T*6*D)); adaln_bias [S*T*6*D] (NULL = 0);
 *           adaln_table [G, r].
 *   SIGLIP: norm1/ln1_b, norm2/ln2_b [D] LayerNorm gain/bias; w_qkv [3D, D]
 *           + b_qkv [3D]; w_out + b_out; w_fc1 [F, D] + b_fc1 [F];
 *           w_fc2 [D, F] + b_fc2 [D].
 *   ZIMAGE: norm1 (attention pre-norm), post_attn_norm, norm2 (FFN pre-norm),
 *           post_ffn_norm [D]; w_qkv, w_out, q_norm, k_norm; w_fc1 [2F, D]
 *           (rows W1 gate | W3 up); w_fc2 [D, F]; temb_w1 [Th, Tf] + temb_b1;
 *           temb_w2 [Tf, Th] + temb_b2; ada_w [4D, Tf] + ada_b [4D]
 *           (chunks scale_msa, gate_msa, scale_mlp, gate_mlp).
 *   REFINER: as MMH3 without the adaLN tensors.
 *   ZCONTEXT: as ZIMAGE without the timestep and adaLN tensors.
 *   ZFINAL: w_fc1 [F, D] output projection + b_fc1 [F] (NULL = 0); temb_w1,
 *           temb_b1, temb_w2, temb_b2 as ZIMAGE; ada_w [D, Tf] + ada_b [D].
 *   rope_freq [rope_axes[0] / 2]: the shared frequency vector of DIT_ROPE_PARTIAL
 *           (MMH3, REFINER), NULL otherwise.
 *   adaln_shared = 1: adaln_basis [T*E*D, r] and adaln_bias [T*E*D] (one slot).
 *   FINAL:  norm1 [D] final RMSNorm gain; w_fc1 [F, D] head weight + b_fc1 [F]
 *           (NULL = 0); adaln_basis [S*2*D, r] (chunk 0 shift, 1 scale per
 *           slot), adaln_bias [S*2*D] (NULL = 0), adaln_table [G, r]. */
typedef struct dit_weights {
  const float *norm1, *norm2, *ln1_b, *ln2_b, *post_attn_norm, *post_ffn_norm;
  const void *w_qkv, *w_out, *w_fc1, *w_fc2;
  const float *b_qkv, *b_out, *b_fc1, *b_fc2;
  const float *q_norm, *k_norm;
  const float *adaln_basis, *adaln_bias, *adaln_table;
  const float *temb_w1, *temb_b1, *temb_w2, *temb_b2, *ada_w, *ada_b;
  const float *rope_freq;
} dit_weights;

/* Byte offsets of the intermediates inside the workspace of dit_block_forward
 * (for inspection after the call; `none` = SIZE_MAX when a variant has no such
 * buffer).  ldn = n rounded up to 128.  act = the config's dtype.
 *   mods  fp32 [R, E*D]   R = S*T (MMH3) or 1 (ZIMAGE), E = 6 or 4 (none: SIGLIP, REFINER)
 *   rope  fp32 [n, hd/2, 2] (cos, sin) per token and pair (DIT_ROPE_PARTIAL: pairs
 *                         [3k, hd/2) hold the identity (1, 0))
 *   xn    act  [n, D]     pre-norm + modulate of the FFN half after the call
 *                         (the attention half's is overwritten)
 *   qkv   act  [n, 3D]    QKV projection (+ bias); fp32 configurations only (the bf16
 *                         QKV GEMM writes q, k and vt directly from its epilogue)
 *   q, k  act  [H, ldn, hd]  after qk-norm and RoPE; q carries log2(e) * hd^-1/2.
 *                         DIT_ROPE_PARTIAL runs as a split-half rotation over all of
 *                         hd with the head dims of q and k permuted (scores are
 *                         unchanged): with P = 3k, h = hd/2, stored dim d holds the
 *                         page's dim d (d < P), d + P (P <= d < h), d - (h - P)
 *                         (h <= d < h + P) or d (d >= h + P)
 *   vt    act  [H, hd, ldn]  V transposed per head
 *   o     act  [n, D]     attention output, head h at columns h*hd
 *   x1    fp32 [n, D]     residual stream after the attention half
 *   a     act  [n, F]     FFN activation (SwiGLU or GELU-tanh)
 *   y     fp32 [n, D]     ZIMAGE: last projection before its sandwich norm (fc2's after the call)
 *   part  fp32            bf16 only: scratch shared by the attention's split tail
 *                         (key-range partials, 256 slots x 256 queries x (hd + 2)
 *                         floats) and the GEMMs' split-K tails (up to 256 slots of
 *                         256 x 256 accumulators); max of the two, contents undefined */
typedef struct dit_ws_layout {
  size_t mods, rope, xn, qkv, q, k, vt, o, x1, a, y, temb, part, total;
  int32_t ldn;
} dit_ws_layout;

/* Checks a configuration; DIT_OK if the library supports it. */
dit_status dit_validate_config(const dit_config* cfg);

/* Bytes of the prepared-weights buffer for `cfg` (0 if cfg is invalid). */
size_t dit_prepared_size(const dit_config* cfg);

/* Copies the raw weights into `prepared` (device, `bytes` long) in the
 * kernels' layout: SwiGLU fc1 rows interleaved in groups of 32 (gate group g,
 * then up group g), SIGLIP W_q and b_q pre-multiplied by hd^-1/2
 * ([SIGLIP] Layer::load, the scale fold).  `raw` may be freed after the
 * stream has passed this call. */
dit_status dit_prepare_weights(const dit_config* cfg, const dit_weights* raw, void* prepared,
                               size_t bytes, void* stream);

/* Workspace bytes needed by dit_block_forward for n tokens. */
size_t dit_workspace_size(const dit_config* cfg, int32_t n);

/* Fills `out` (host) with the workspace layout for n tokens. */
dit_status dit_workspace_layout(const dit_config* cfg, int32_t n, dit_ws_layout* out);

/* Modulation rows ([MMH3] Adaln::eval; [ZIMG] TimestepEmbedder + adaLN).
 * sigmas (host, n_sigmas = S for MMH3, 1 for ZIMAGE):
 *   MMH3:   slot s's sigma; t_s = 1 - sigma_s as given (no floor: a slot
 *           sigma of 0 is t = 1, which reads table row G-1 with weight 1),
 *           grid coordinate p = clamp(t_s, 0, 1)*(G-1) taken in fp64 on the
 *           host; row j of the basis is evaluated at its own slot's
 *           interpolated coordinates.  The evaluation's 1e-6 floor of the
 *           video sigma is dit_mmh3_slots'.
 *   ZIMAGE: sigmas[0] is the timestep t (multiplied by t_scale).
 * mods_out: device fp32 [R, E*D], element (r, e, d) at (r*E + e)*D + d.
 * temb_scratch: ZIMAGE only, device fp32 [temb_hidden + temb_freq] (else NULL). */
dit_status dit_adaln_eval(const dit_config* cfg, const void* prepared, const double* sigmas,
                          int32_t n_sigmas, float* mods_out, float* temb_scratch, void* stream);

/* dit_adaln_eval without the scratch argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments and result as
 * dit_adaln_eval; the Z-Image timestep MLP's scratch (temb_hidden + temb_freq
 * floats) is a library-owned device array of DIT_NOALLOC_TEMB_MAX floats per
 * GPU, held until the process ends.  A configuration needing more is refused
 * with DIT_EUNSUPPORTED before anything is launched.  The array is shared by
 * every call on one GPU: calls that overlap on one GPU (other streams or
 * threads) race on it and must be ordered by the caller.  MMH3 and FINAL
 * configurations use no scratch.  Allocates nothing. */
#define DIT_NOALLOC_TEMB_MAX 16384
dit_status dit_adaln_eval_noalloc(const dit_config* cfg, const void* prepared,
                                  const double* sigmas, int32_t n_sigmas, float* mods_out,
                                  void* stream);

/* Modulation + segment gather + pre-norm + modulate of one half of the block:
 * mods_out = dit_adaln_eval(...), then for every token i with r = rows[i]:
 *   MMH3:   xn_i = RMSNorm(x_i; g, eps) * (1 + mods[r, scale]) + mods[r, shift]
 *           (half 0: g = norm1, chunks shift 0 / scale 1; half 1: norm2, 3 / 4)
 *   ZIMAGE: xn_i = RMSNorm(x_i; g, eps) * (1 + mods[0, scale]) (chunk 0 or 2)
 *   SIGLIP: xn_i = LayerNorm(x_i; g, b, eps), mods unused (may be NULL)
 *   REFINER: xn_i = RMSNorm(x_i; g, eps), mods unused (may be NULL)
 * x: device fp32 [n, D]; rows: device int32 [n], each in [0, R) (unchecked on
 * the device: an out-of-range row reads outside mods); NULL means row 0.
 * xn_out: device [n, D] in the config's dtype. */
dit_status dit_adaln_modulate(const dit_config* cfg, const void* prepared, const float* x,
                              int32_t n, const int32_t* rows, const double* sigmas,
                              int32_t n_sigmas, int32_t half, void* xn_out, float* mods_out,
                              float* temb_scratch, void* stream);

/* One block forward ([MMH3] block_forward + ffn_tail; [SIGLIP] Layer::forward;
 * [ZIMG] TransformerBlock.Forward):
 *   x:    device fp32 [n, D] residual stream in
 *   rows: device int32 [n] modulation row per token (MMH3; NULL = row 0)
 *   pos:  device fp32 [n, 3] (t, h, w) per token (needed unless rope = NONE)
 *   sigmas: host, as dit_adaln_eval (ignored for SIGLIP and REFINER)
 *   out:  device fp32 [n, D]; may alias x (x is read only before out is written)
 *   workspace: device, >= dit_workspace_size(cfg, n) bytes, 256-byte aligned */
dit_status dit_block_forward(const dit_config* cfg, const void* prepared, const float* x,
                             int32_t n, const int32_t* rows, const float* pos,
                             const double* sigmas, int32_t n_sigmas, float* out,
                             void* workspace, size_t ws_bytes, void* stream);

/* Several independent samples packed in one sequence ([ENC] attention_ragged
 * over seq_starts: each query attends only to the keys of its own sample, so
 * the packed call equals the samples run one by one; every other step of the
 * block is per token).  seq_starts: HOST int32 [nseq + 1], seq_starts[0] = 0,
 * non-decreasing (empty samples allowed), seq_starts[nseq] = n, 1 <= nseq <=
 * DIT_MAX_SEQS; refused with DIT_ESHAPE otherwise.  Positions and rows are the
 * caller's per token (a sample's positions are its own).  Arguments otherwise as
 * dit_block_forward; nseq = 1 computes exactly what dit_block_forward does. */
#define DIT_MAX_SEQS 64
dit_status dit_block_forward_packed(const dit_config* cfg, const void* prepared, const float* x,
                                    int32_t n, const int32_t* rows, const float* pos,
                                    const double* sigmas, int32_t n_sigmas,
                                    const int32_t* seq_starts, int32_t nseq, float* out,
                                    void* workspace, size_t ws_bytes, void* stream);

/* dit_block_forward with the modulation rows supplied instead of evaluated
 * (MMH3 and ZIMAGE; refused with DIT_EUNSUPPORTED for the others): for rows
 * from another source, e.g. a full-rank adaLN map, or one basis shared by
 * every timestep as [MMH3] Adaln::eval evaluates it, or rows evaluated once and
 * reused across calls.
 *   mods: device fp32 [R, E*D] in dit_adaln_eval's layout (read only);
 *   seq_starts/nseq: as dit_block_forward_packed, or NULL for one sequence.
 * With mods from dit_adaln_eval(sigmas) this computes exactly what
 * dit_block_forward(sigmas) computes. */
dit_status dit_block_forward_mods(const dit_config* cfg, const void* prepared, const float* x,
                                  int32_t n, const int32_t* rows, const float* pos,
                                  const float* mods, const int32_t* seq_starts, int32_t nseq,
                                  float* out, void* workspace, size_t ws_bytes, void* stream);

/* Output head of the MMH3 model (config variant DIT_FINAL; [MMH3]
 * MiniMaxH3::forward, "heads"): with the rows m = dit_adaln_eval(sigmas)
 * [S, 2D] of the head's own rank-r basis,
 *   out_i = -(W (RMSNorm(h_i; g, eps) * (1 + m[r, D:2D]) + m[r, 0:D]) + b)
 * for r = rows[i] (the token's timestep slot; NULL = 0).  h: device fp32
 * [n, D]; out: device fp32 [n, F]; workspace: dit_workspace_size(cfg, n).
 * With a DIT_ZFINAL config (the Z-Image final layer, one sigma = its t):
 *   out_i = W (LayerNorm_noaffine(h_i; eps) * (1 + scale)) + b,
 *   scale = ada_w silu(temb(t * t_scale)) + ada_b  (rows unused). */
dit_status dit_final_forward(const dit_config* cfg, const void* prepared, const float* h,
                             int32_t n, const int32_t* rows, const double* sigmas,
                             int32_t n_sigmas, float* out, void* workspace, size_t ws_bytes,
                             void* stream);

/* out[m, nout] = alpha * (a[m, k] . w[nout, k]^T + bias), the embedding and
 * head projections around the blocks, on the block GEMM kernels.  a and w in
 * dtype (row-major, lda >= k), bias fp32 [nout] or NULL, out fp32 [m, nout].
 * bf16: k % 64 == 0, nout % 32 == 0; fp32: k % 16 == 0, nout % 64 == 0;
 * 16-byte aligned pointers; refused with DIT_EUNSUPPORTED / DIT_EALIGN. */
dit_status dit_linear(int32_t dtype, const void* a, int32_t lda, int32_t m, int32_t k,
                      const void* w, int32_t nout, const float* bias, float alpha, float* out,
                      void* stream);

/* Latent streams <-> token rows ([MMH3] patchify_video, unpatchify_video,
 * pack_audio, unpack_audio).  video: device fp32 [C, T, H, W] (H, W even);
 * rows [T*(H/2)*(W/2), 4C], row (t, h2, w2) holding the 2 x 2 patch at
 * (2*h2, 2*w2) of frame t, column c*4 + p*2 + q = x[c, t, 2*h2 + p, 2*w2 + q].
 * audio: device fp32 [C, 2, T]; rows [2T, C], row ch*T + t, column c =
 * x[c, ch, t].  The packing side writes rows in `dtype` (the embedding GEMM's
 * operand); the unpacking side reads fp32 rows (the head's output). */
dit_status dit_patchify_video(int32_t dtype, const float* x, int32_t C, int32_t T, int32_t H,
                              int32_t W, void* rows, void* stream);
dit_status dit_unpatchify_video(const float* rows, int32_t C, int32_t T, int32_t H, int32_t W,
                                float* x, void* stream);
dit_status dit_pack_audio(int32_t dtype, const float* x, int32_t C, int32_t T, void* rows,
                          void* stream);
/* The Z-Image patch layout ([ZIMG] PatchifyLatents / UnpatchifyLatents):
 * image device fp32 [C, H, W] (H, W even) <-> rows [(H/2)*(W/2), 4C], row
 * (h2, w2), column (p*2 + q)*C + c = x[c, 2*h2 + p, 2*w2 + q] (channel fastest). */
dit_status dit_patchify_image(int32_t dtype, const float* x, int32_t C, int32_t H, int32_t W,
                              void* rows, void* stream);
dit_status dit_unpatchify_image(const float* rows, int32_t C, int32_t H, int32_t W, float* x,
                                void* stream);
dit_status dit_unpack_audio(const float* rows, int32_t C, int32_t T, float* x, void* stream);

/* One denoise evaluation of the MMH3 model ([MMH3] MiniMaxH3::forward):
 * embed (video and condition frames through the video patch projection, audio
 * through the audio one, refined text copied in), the timestep slots of
 * dit_mmh3_slots and the token rows, the blocks in order, then the video and
 * audio heads (dit_final_forward, negated) and the unpacking of their rows.
 * Condition latents are taken as given (any noise augmentation is the
 * caller's); the text span carries the text tag unless per-token tags are
 * given. */
typedef enum {
  DIT_SEG_TEXT = 0,
  DIT_SEG_VIDEO = 1,      /* the noisy target, T*(H/2)*(W/2) rows */
  DIT_SEG_AUDIO = 2,      /* 2*Ta rows */
  DIT_SEG_COND = 3,       /* one condition frame, (H/2)*(W/2) rows */
  DIT_SEG_REF_IMAGE = 4,  /* layout only: a reference image, or a reference clip's frames */
  DIT_SEG_REF_AUDIO = 5   /* layout only: reference audio, or a reference clip's soundtrack */
} dit_segment_kind;
/* dit_mmh3_forward refuses the two reference kinds: [MMH3] MiniMaxH3::forward
 * plans their slots and rows (see dit_mmh3_slots) but embeds no hidden rows for
 * them; a caller that embeds references runs the blocks with dit_stack_forward. */

typedef struct dit_segment {
  int32_t kind, start, stop; /* rows [start, stop) of the packed sequence */
} dit_segment;

typedef struct dit_mmh3_model {
  const dit_config* block;          /* DIT_MMH3; slots >= the slots of an evaluation (<= 3) */
  const void* const* blocks;        /* n_blocks prepared block weights (host array)        */
  int32_t n_blocks;
  const dit_config* head_video;     /* DIT_FINAL, F = 4 * latent_c, same slots as block     */
  const void* head_video_w;         /* prepared                                            */
  const dit_config* head_audio;     /* DIT_FINAL, F = audio_c                               */
  const void* head_audio_w;
  int32_t latent_c, audio_c;        /* latent channels of the video and audio streams     */
  const void* video_patch_w;        /* [D, 4*latent_c] in the block dtype                  */
  const float* video_patch_b;       /* [D] or NULL                                          */
  const void* audio_patch_w;        /* [D, audio_c] in the block dtype                     */
  const float* audio_patch_b;       /* [D] or NULL                                          */
  double shift_video, shift_audio;  /* flow shifts (12, 3)                                  */
  double cond_aug, cond_aug_audio;  /* condition timesteps (0.999, 1)                       */
  int32_t audio_slope_rescale;      /* 0: both velocities unscaled, each on its own schedule;
                                       1: the audio velocity times d(sigma_a)/d(sigma_v) =
                                       dit_sigma_remap_slope(sigma_v, shift_video, shift_audio),
                                       the single-schedule form [MMH3] ascribes to the
                                       reference model                                     */
} dit_mmh3_model;

/* The packed layout of one evaluation ([MMH3] Layout::t2va / fl2va / ref2va):
 * segments in order [text | references | keyframes | audio | video] and every
 * row's (t, h, w) position, in fp64 as the page keeps them.
 *   text token i at (i, 0, 0); the cursor starts at text_len;
 *   the h and w axes of a lat_h x lat_w latent are the dim/2 points
 *     32 * ((1 - r)/2 + i * r / (dim/2)), r = dim / sqrt(lat_h * lat_w);
 *   references (refs, in order) advance the cursor: an image by 1 (its own
 *     grid, one time step); an audio block by its frames (stereo at the
 *     target's w extremes); a clip packs its soundtrack (its own grid's w
 *     extremes) then its frames from the cursor and advances by the longer;
 *   keyframes (pairs pixel_index, frame_count: the clip's first frame, at the
 *     cursor, or its last, at cursor + all frame spans - 5/3) share the target
 *     grid and do not advance the cursor;
 *   audio: 2 * audio_t rows, channel-major, (cursor + i, 0, w_lo) then
 *     (cursor + i, 0, w_hi); video: latent_t frames of the target grid from
 *     the cursor, t advancing by 5/3 * (1, 4, 4, 4, 4)[k % 5].
 * Host function.  lat_h, lat_w >= 2 (refs likewise).  Returns the row count
 * and sets *n_segs; with pos == NULL only counts.  pos: [max_rows, 3];
 * segs: [max_segs].  Errors (negative): DIT_EINVAL for a keyframe that is not
 * a first or last frame, an unknown reference kind or a failed host
 * allocation, DIT_ESHAPE for sizes, a layout of more than 2^24 rows or
 * too-small outputs. */
typedef struct dit_layout_ref {
  int32_t kind;  /* DIT_SEG_REF_IMAGE (lat_h, lat_w), DIT_SEG_REF_AUDIO (audio_t) or
                    DIT_SEG_VIDEO for a reference clip (latent_t, lat_h, lat_w, audio_t) */
  int32_t latent_t, lat_h, lat_w, audio_t;
} dit_layout_ref;

int32_t dit_mmh3_layout(int32_t text_len, int32_t latent_t, int32_t lat_h, int32_t lat_w,
                        int32_t audio_t, const int32_t* keyframes, int32_t n_keyframes,
                        const dit_layout_ref* refs, int32_t n_refs, double* pos, int32_t max_rows,
                        dit_segment* segs, int32_t max_segs, int32_t* n_segs);

/* Workspace bytes of dit_mmh3_forward for these segments (0 if invalid). */
size_t dit_mmh3_workspace_size(const dit_mmh3_model* m, const dit_segment* segs, int32_t nseg);

/* segs: host, nseg entries covering [0, n) without gaps; one VIDEO, at most one
 * AUDIO, one TEXT, any number of COND.  pos: device fp32 [n, 3].  text:
 * device fp32 [text rows, D] (refined).  video: device fp32 [latent_c, T, H, W];
 * text_tags: device int32 [text rows], each token's modality tag (0 video, 1
 * text, 2 audio: a vision block inside the prompt carries the video tag,
 * [MMH3] Layout text_tags), clamped to [0, 2]; NULL = every token text.
 * audio: device fp32 [audio_c, 2, Ta] (NULL without an AUDIO segment).  cond:
 * host array of device pointers, one fp32 [latent_c, 1, H, W] per COND segment
 * in order.  Outputs (device fp32, same shapes as the inputs): the video and
 * audio velocities.  The embedding GEMMs need a depth multiple of 64 (bf16) or
 * 16 (fp32): latent_c % 16 == 0 and audio_c % 64 == 0 for bf16 blocks,
 * latent_c % 4 == 0 and audio_c % 16 == 0 for fp32 blocks. */
dit_status dit_mmh3_forward(const dit_mmh3_model* m, const dit_segment* segs, int32_t nseg,
                            const float* pos, const float* text, const int32_t* text_tags,
                            const float* video, int32_t T,
                            int32_t H, int32_t W, const float* audio, int32_t Ta,
                            const float* const* cond, double sigma_v, float* video_out,
                            float* audio_out, void* workspace, size_t ws_bytes, void* stream);

/* The Z-Image transformer ([ZIMG] Transformer.Forward / ForwardWithCache). */
typedef struct dit_zimage_model {
  const dit_config* block;            /* DIT_ZIMAGE: main layers and noise refiners      */
  const void* const* layers;          /* n_layers prepared main layers (host array)      */
  int32_t n_layers;
  const void* const* noise_refiners;  /* image tokens only, modulated                    */
  int32_t n_noise_refiners;
  const dit_config* context;          /* DIT_ZCONTEXT, same D/H/hd as block (may be NULL
                                         with no context refiners)                       */
  const void* const* context_refiners;/* caption tokens only, unmodulated                */
  int32_t n_context_refiners;
  const dit_config* final_layer;      /* DIT_ZFINAL, F = 4 * in_channels                 */
  const void* final_w;
  int32_t in_channels, cap_dim;
  const void* x_embed_w;              /* [D, 4 * in_channels] in the block dtype         */
  const float* x_embed_b;             /* [D] or NULL                                     */
  const float* cap_norm;              /* [cap_dim] RMSNorm gain of the caption embedder  */
  float cap_eps;                      /* its epsilon (1e-6)                              */
  const void* cap_embed_w;            /* [D, cap_dim] in the block dtype                 */
  const float* cap_embed_b;           /* [D] or NULL                                     */
} dit_zimage_model;

/* Step-level reuse state ([ZIMG] ForwardWithCache), caller-owned.  caption:
 * device fp32 [cap_len, D], the embedded and refined caption, computed on the
 * first call and reused while caption_valid (it depends on neither t nor the
 * latents).  shallow: device fp32 [img_len + cap_len, D], the unified stream
 * after the first `layers` main layers, stored on refresh steps (step %
 * interval == 0) and reused on the others; a reused step skips the image
 * embedding, the noise refiners and those layers, whose results the stored
 * stream replaces.  The valid flags are set by dit_zimage_forward when it
 * enqueues the stores; set both to 0 for a new generation.  Calls that share
 * a cache must run in stream order. */
typedef struct dit_zimage_cache {
  float* caption;
  float* shallow;
  int32_t layers;    /* shallow layers, 0 <= layers <= n_layers (0: no layer reuse) */
  int32_t interval;  /* >= 1 */
  int32_t caption_valid, shallow_valid;
} dit_zimage_cache;

/* Workspace bytes of dit_zimage_forward (0 if invalid). */
size_t dit_zimage_workspace_size(const dit_zimage_model* m, int32_t H, int32_t W, int32_t cap_len);

/* latents: device fp32 [in_channels, H, W]; cap_feats: device fp32 [cap_len,
 * cap_dim]; pos: device fp32 [img_len + cap_len, 3], image tokens first (the
 * unified order; the refiners read their own parts); t: the timestep (the
 * blocks embed t * t_scale); cache: NULL computes everything.  out: device
 * fp32 [in_channels, H, W], the final layer's output unpatchified.  The
 * embedding GEMMs need 4 * in_channels and cap_dim to be multiples of 64
 * (bf16) or 16 (fp32); cap_dim <= 4096. */
dit_status dit_zimage_forward(const dit_zimage_model* m, const float* latents, int32_t H, int32_t W,
                              const float* cap_feats, int32_t cap_len, const float* pos, double t,
                              int32_t step, dit_zimage_cache* cache, float* out, void* workspace,
                              size_t ws_bytes, void* stream);

/* RMSNorm of fp32 rows into fp32 rows: out_i = x_i / sqrt(mean(x_i^2) + eps) * g
 * (e.g. the token refiner's final norm, [MMH3] refine_text).  D % 4 == 0,
 * D <= 4096, 16-byte aligned pointers; out may alias x. */
dit_status dit_rms_norm(const float* x, int32_t n, int32_t D, const float* g, float eps, float* out,
                        void* stream);

/* A stack of n_blocks blocks of one configuration, in order, each with its own
 * prepared weights (prepared[i], device): out = block_{L-1}(... block_0(x)),
 * all blocks with the same rows, positions, sigmas and packed-sample table
 * (seq_starts may be NULL).  The intermediate residual stream lives in out
 * (out may alias x); workspace as for one block. */
dit_status dit_stack_forward(const dit_config* cfg, const void* const* prepared, int32_t n_blocks,
                             const float* x, int32_t n, const int32_t* rows, const float* pos,
                             const double* sigmas, int32_t n_sigmas, const int32_t* seq_starts,
                             int32_t nseq, float* out, void* workspace, size_t ws_bytes,
                             void* stream);

/* Standalone full bidirectional attention over one packed sequence, per head
 * ([MMH3] attention; online softmax with normalization deferred to the output,
 * [SIGLIP] deferred normalisation):
 *   q, k: device [H, ldn, hd]; vt: device [H, hd, ldn] (V transposed), all in
 *   the config's dtype, rows/columns >= n ignored (keys are masked, but the
 *   padding of vt must hold finite values);
 *   o: device [n, H*hd] in the config's dtype;
 *   score_scale: multiplier of q.k before the softmax (q is used as given).
 * ldn must be a multiple of 128 and >= n. */
dit_status dit_attention(const dit_config* cfg, const void* q, const void* k, const void* vt,
                         int32_t n, int32_t ldn, float score_scale, void* o, void* stream);

/* dit_attention with the samples of seq_starts (host, as in
 * dit_block_forward_packed): query i attends to the keys of its own sample. */
dit_status dit_attention_packed(const dit_config* cfg, const void* q, const void* k,
                                const void* vt, int32_t n, int32_t ldn,
                                const int32_t* seq_starts, int32_t nseq, float score_scale,
                                void* o, void* stream);

/* One GPU's share of the attention of a token-sharded sequence: the queries of
 * tokens [qlo, qhi) against all n keys of one sequence (the state after the
 * keys and values of every shard have been gathered; [MMH3] attention, every
 * token attends to every token, run for a contiguous range of query tokens).
 *   q: device [H, ldq, hd], row r = token qlo + r (rows >= qhi - qlo ignored);
 *   k: device [H, ldn, hd]; vt: device [H, hd, ldn] (V transposed), as in
 *   dit_attention;
 *   o: device [qhi - qlo, H*hd], row r = token qlo + r; all in the config's dtype;
 *   workspace: device, 256-byte aligned, at least
 *   dit_attention_shard_workspace_size(cfg) bytes (key-range partials of the
 *   grid's split last round; 0 bytes, and NULL allowed, for fp32).
 * 0 <= qlo <= qhi <= n <= ldn, ldn % 128 == 0, qhi - qlo <= ldq, ldq % 128 == 0.
 * Row r of o equals row qlo + r of dit_attention's o over the whole sequence up
 * to rounding order.  Errors: DIT_ESHAPE for the ranges, DIT_EALIGN,
 * DIT_EWORKSPACE, DIT_EINVAL (NULL pointers, a non-finite score_scale). */
size_t dit_attention_shard_workspace_size(const dit_config* cfg);
dit_status dit_attention_shard(const dit_config* cfg, const void* q, int32_t ldq, int32_t qlo,
                               int32_t qhi, const void* k, const void* vt, int32_t n,
                               int32_t ldn, float score_scale, void* o, void* workspace,
                               size_t ws_bytes, void* stream);

/* Per-phase timing of dit_block_forward ([MMH3] per-phase profiler: one
 * stopwatch per phase, none overlapping).  dit_profile_begin(max_calls) arms
 * hipEvents (created on the host; no device memory) for the next max_calls
 * block calls on this thread; each call records DIT_NPHASES + 1 events on its
 * stream, one before its first kernel and one after each phase.
 * dit_profile_end() waits for the last recorded event, writes the summed
 * milliseconds of every phase over the recorded calls into phase_ms (host,
 * DIT_NPHASES doubles) and the number of recorded calls into *calls, and
 * releases the events.  Phases: 0 adaLN + RoPE table, 1 pre-norm (attention),
 * 2 QKV GEMM (with qk-norm, RoPE and the head split for bf16), 3 qk-norm/RoPE split
 * (fp32 only; empty for bf16), 4 attention, 5 out GEMM + residual,
 * 6 pre-norm (FFN), 7 fc1 GEMM + activation, 8 fc2 GEMM + residual. */
#define DIT_NPHASES 9
dit_status dit_profile_begin(int32_t max_calls);
dit_status dit_profile_end(double* phase_ms, int32_t* calls);
const char* dit_phase_name(int32_t phase);

/* sigma on the to_shift flow schedule at the same base-grid point as sigma on
 * the from_shift schedule ([MMH3] time_shift_sigma); 12 -> 3 is s / (4 - 3s).
 * Host function. */
double dit_sigma_remap(double sigma, double from_shift, double to_shift);

/* The timestep slots of one MMH3 evaluation ([MMH3] MiniMaxH3::forward): the
 * video stream at t_v = 1 - max(sigma_v, 1e-6), the audio stream at t_a =
 * 1 - dit_sigma_remap(max(sigma_v, 1e-6), shift_video, shift_audio), condition
 * frames and reference images (has_cond) at t_c = max(t_v, cond_aug),
 * reference audio (has_ref_audio) at t_ca = max(t_a, cond_aug_audio).  The
 * distinct values, sorted ascending, are the slots (so the order is part of
 * the contract).  Writes slot_sigmas[s] = 1 - t_s, the sigmas that the block
 * entry points take (they evaluate slot s at 1 - sigma: the reference-audio
 * slot at t = 1 exactly reads the adaLN table's last row), and slot_of = {video, audio, cond,
 * ref audio} slot indices (-1 when absent).  A token's modulation row is then
 * slot * 3 + tag (video 0, text 1, audio 2; condition frames and reference
 * images take the video tag, reference audio the audio tag).  Host function;
 * returns the slot count (1..4), or DIT_EINVAL for non-finite input, a flow
 * shift <= 0 or a remapped audio sigma that is not finite. */
int32_t dit_mmh3_slots(double sigma_v, double shift_video, double shift_audio, double cond_aug,
                       double cond_aug_audio, int32_t has_cond, int32_t has_ref_audio,
                       double slot_sigmas[4], int32_t slot_of[4]);

/* d sigma_to / d sigma_from of dit_sigma_remap ([MMH3] time_shift_slope). */
double dit_sigma_remap_slope(double sigma, double from_shift, double to_shift);

/* Message of the last failure on this thread ("" if none). */
const char* dit_last_error(void);

/* ABI version (increments on any change of this header). */
int32_t dit_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DIT_H */
