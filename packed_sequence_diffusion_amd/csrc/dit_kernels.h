// Launchers of the block's HIP kernels (internal to libdit.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

enum Dtype { F32 = 0, BF16 = 1 };

// ---- GEMM: C[M, N] = A[M, K] * B[N, K]^T with a fused epilogue ----------------
enum EpiKind {
  EPI_STORE = 0,      // out[r, c] = acc (+ bias[c])
  EPI_GATED_RES = 1,  // out_f32[r, c] = resid[r, c] + gate(r, c) * (acc (+ bias[c])); gate = 1 without mods
  EPI_SWIGLU = 2,     // columns interleaved in groups of 32 (gate g, up g): out[r, c'] = silu(g) * u
  EPI_GELU = 3,       // out[r, c] = gelu_tanh(acc + bias[c])
  EPI_QKV = 4         // bf16 QKV head split: (+ bias), qk-RMSNorm, RoPE and the q scale on
                      // q and k, written head-major [H, ldn, hd]; v written transposed
                      // [H, hd, ldn]; rows in [M, ldn) written as zeros
};

struct Epi {
  void* out = nullptr;  // element type: fp32 for GATED_RES, else the GEMM's out type
  int ldc = 0;
  const float* bias = nullptr;   // [N] (GELU, STORE, GATED_RES) or null
  float alpha = 1.0f;            // STORE: out = alpha * (acc + bias)
  const float* resid = nullptr;  // GATED_RES: fp32 [M, ldr]
  int ldr = 0;
  const float* mods = nullptr;  // GATED_RES: gate = mods[rows[r] * mstride + goff + c]
  int mstride = 0;
  int goff = 0;
  const int* rows = nullptr;  // null = row 0
  // EPI_QKV (ldc holds D = H * hd)
  int hd = 0, ldn = 0;
  const float* qn = nullptr;  // q_norm / k_norm gains [hd], null = no qk-norm
  const float* kn = nullptr;
  float qk_eps = 0.0f;
  const float* cs = nullptr;  // RoPE (cos, sin) [M, hd/2, 2]
  int rope = 0;               // 0 none, 1 split-half, 2 interleaved
  float q_scale = 1.0f;
  void* q = nullptr;
  void* k = nullptr;
  void* vt = nullptr;
  // bf16: scratch of gemm_split_bytes() for a split-K tail (null: no split)
  float* split = nullptr;
};

// Scratch a bf16 GEMM may use for its split-K tail: at most kGemmSplitWgs
// workgroups, each with one fp32 256 x 256 accumulator tile.
constexpr int kGemmSplitWgs = 256;
inline size_t gemm_split_bytes() { return (size_t)kGemmSplitWgs * 256 * 256 * sizeof(float); }

hipError_t gemm(int dtype, int epi, bool out_bf16, const void* A, int lda, const void* B, int ldb,
                int M, int N, int K, const Epi& ep, hipStream_t s);

// ---- modulation --------------------------------------------------------------------
struct SlotCoords {
  int i0[8];
  float f[8];
};
hipError_t adaln_interp(const float* basis, const float* bias, const float* table, int rank,
                        int per_slot, int slots, const SlotCoords& sc, float* mods, hipStream_t s);
// Z-Image: sinusoid(t) -> L1 + SiLU -> L2 -> adaLN linear; scratch [hidden + freq].
hipError_t temb_mods(double t_scaled, int freq, int hidden, int out_dim, const float* w1,
                     const float* b1, const float* w2, const float* b2, const float* wa,
                     const float* ba, float* scratch, float* mods, hipStream_t s,
                     bool silu_temb = false);

// ---- row kernels --------------------------------------------------------------------
enum NormKind { NORM_RMS = 0, NORM_LAYER = 1 };
enum ModKind { MOD_NONE = 0, MOD_SHIFT_SCALE = 1, MOD_SCALE = 2 };
hipError_t norm_mod(int norm, int mod, bool out_bf16, const float* x, int n, int D, const float* g,
                    const float* beta, float eps, const float* mods, int mstride, const int* rows,
                    int shift_off, int scale_off, void* y, hipStream_t s);

// x1 = x + tanh(gate) * RMSNorm(y; g_post); optionally xf = RMSNorm(x1; g_next) * (1 + scale).
hipError_t sandwich(const float* x, const float* y, int n, int D, const float* g_post,
                    const float* gate, float eps, float* x1, const float* g_next,
                    const float* scale, bool xf_bf16, void* xf, hipStream_t s);

// cos/sin per token and rotation pair, from fp64 angles.
hipError_t rope_table_shared(const float* pos, int n, int P, int k, const float* freq, float* cs,
                             hipStream_t s);
hipError_t rope_table(const float* pos, int n, int P, const int axes[3], double theta, float* cs,
                      hipStream_t s);

// qkv [n, 3D] -> q, k [H, ldn, hd] (qk-norm, RoPE, q scaled), vt [H, hd, ldn]; rows >= n zero.
hipError_t qk_split(int dtype, int hd, const void* qkv, int n, int ldn, int H, const float* qn,
                    const float* kn, float eps, const float* cs, int rope_mode, float q_scale,
                    void* q, void* k, void* vt, hipStream_t s);

// Attention over all n keys per head; q carries the base-2 score scale times
// scale_log2.  bf16: `part` (attention_part_bytes(hd), may be null) holds the
// key-range partials of the grid's last, split round; null disables the split.
constexpr int kAttnMaxSlots = 256;  // split workgroups in the last round, at most
constexpr int kAttnQueryRows = 256; // queries per workgroup
inline size_t attention_part_bytes(int hd) {
  return (size_t)kAttnMaxSlots * kAttnQueryRows * (size_t)(hd + 2) * sizeof(float);
}
// Independent samples packed in one sequence: sample s is tokens
// [start[s], start[s+1]) and its queries attend only to its own keys.
// blk[s] = query blocks of kAttnQueryRows before sample s (blk[nseq] = total).
// Passed by value to the kernels.
constexpr int kMaxSeqs = 64;
// With one sample, the queries may be a contiguous range [qlo, qhi) of its
// tokens (one GPU's share of a token-sharded sequence: the queries of that
// range against every key); q and o then hold those queries only, row r being
// token qbase + r.  Otherwise qlo = 0, qhi = n, qbase = 0.
struct SeqTable {
  int nseq;
  int start[kMaxSeqs + 1];
  int blk[kMaxSeqs + 1];
  int qlo, qhi, qbase;
};
// Builds the table from host offsets (nullptr: one sequence of n tokens).
void make_seq_table(const int* seq_starts, int nseq, int n, SeqTable* t);
// One sequence of n tokens whose queries are the tokens [qlo, qhi).
void make_shard_table(int n, int qlo, int qhi, SeqTable* t);
// q: [H, ldq, hd] (ldq = ldn without a query range), k: [H, ldn, hd], vt: [H, hd, ldn].
hipError_t attention(int dtype, int hd, const void* q, int ldq, const void* k, const void* vt,
                     int n, int ldn, int H, float scale_log2, void* o, float* part,
                     const SeqTable& seqs, hipStream_t s);

// ---- latent streams <-> token rows (k_streams.hip) --------------------------------------
hipError_t patchify_video(int dtype, const float* x, int C, int T, int H, int W, void* rows,
                          hipStream_t s);
hipError_t unpatchify_video(const float* rows, int C, int T, int H, int W, float* x, hipStream_t s);
hipError_t pack_audio(int dtype, const float* x, int C, int T, void* rows, hipStream_t s);
hipError_t unpack_audio(const float* rows, int C, int T, float* x, hipStream_t s);
// channel-last patch columns ([ZIMG] PatchifyLatents), image [C, H, W]
hipError_t patchify_image(int dtype, const float* x, int C, int H, int W, void* rows, hipStream_t s);
hipError_t unpatchify_image(const float* rows, int C, int H, int W, float* x, hipStream_t s);
// p[0, n) = v (a kernel rather than a memset: safe inside captured graphs)
hipError_t fill_i32(int* p, int n, int v, hipStream_t s);
// compute units of the current device (cached per device; 256 if the query fails)
int device_cus();
hipError_t fill_f32(float* p, int n, float v, hipStream_t s);
// rows[i] = base + clamp(tags[i], 0, 2) (per-token modality rows of the prompt span)
hipError_t rows_from_tags(const int* tags, int n, int base, int* rows, hipStream_t s);

// ---- weight preparation ---------------------------------------------------------------
// Source row of prepared row r, in this order: the SwiGLU group interleave (swiglu_F > 0);
// for r < perm_rows, the head-dim permutation that runs the partial split-half RoPE as a
// full one (perm_hd, perm_P = 3k rotated pairs); the source row modulo src_mod (> 0: one
// slot's adaLN rows repeated for every slot).
struct RowMap {
  int swiglu_F = 0;
  int perm_rows = 0, perm_hd = 0, perm_P = 0;
  int src_mod = 0;
};
// dst[r, :] = src[map(r), :] * (r < scale_rows ? scale : 1)
hipError_t prep_matrix(int dtype, const void* src, void* dst, int rows, int cols, const RowMap& m,
                       int scale_rows, float scale, hipStream_t s);
hipError_t prep_matrix(int dtype, const void* src, void* dst, int rows, int cols, int swiglu_F,
                       int scale_rows, float scale, hipStream_t s);
// dst[i] = src[map(i)] * (i < scale_n ? scale : 1) (src NULL: zeros)
hipError_t prep_vector(const float* src, float* dst, int n, const RowMap& m, int scale_n,
                       float scale, hipStream_t s);
hipError_t prep_vector(const float* src, float* dst, int n, int scale_n, float scale,
                       hipStream_t s);

}  // namespace dit
