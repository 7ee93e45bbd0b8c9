// GEMMs of the block, C[M, N] = A[M, K] * B[N, K]^T (both operands K-contiguous,
// weights stored [out, in]), with the epilogues fused into the store:
// plain/bias store, gated residual ([MMH3] residual), SwiGLU pairing ([MMH3]
// ffn_tail) and bias + GELU-tanh ([SIGLIP] GeluBiasOp).
//
// bf16 path: v_mfma_f32_32x32x16_bf16 on LDS-staged 256x256x64 tiles; eight
// waves, each owning a 64x128 strip of the tile (2x4 MFMA blocks of 32x32).
// fp32 path: a plain LDS-tiled FMA kernel (64x64 tiles), used by the fp32
// block configuration.
#include "dev_common.h"
#include "dit_kernels.h"

namespace dit {

// ---------------------------------------------------------------- epilogues ----
template <int EPI, typename OutT>
DIT_DEV void epi_one(const Epi& ep, int row, int col, float v) {
  if (EPI == EPI_STORE) {
    if (ep.bias) v += ep.bias[col];
    Elt<OutT>::st((OutT*)ep.out + (size_t)row * ep.ldc + col, ep.alpha * v);
  } else if (EPI == EPI_GELU) {
    if (ep.bias) v += ep.bias[col];
    Elt<OutT>::st((OutT*)ep.out + (size_t)row * ep.ldc + col, gelu_tanh_f(v));
  }
}

template <typename OutT>
DIT_DEV void epi_swiglu(const Epi& ep, int row, int ocol, float g, float u) {
  Elt<OutT>::st((OutT*)ep.out + (size_t)row * ep.ldc + ocol, silu_f(g) * u);
}

// Gated residual for NV accumulator rows of one lane: out = resid + gate * (acc
// + bias).  All loads are issued before any store (the residual, the gates
// and the output never overlap within one GEMM), so the epilogue pays one
// memory latency instead of one per element.
template <int NR, int NC>
DIT_DEV void epi_gated_rows(const Epi& ep, const int (&row)[NR], int M, int cbase, int cl,
                            const float (&acc)[NR][NC]) {
  const float* __restrict__ resid = ep.resid;
  float* __restrict__ out = (float*)ep.out;
  float rv[NR][NC], gv[NR][NC], bv[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) bv[j] = ep.bias ? ep.bias[cbase + 32 * j + cl] : 0.0f;
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int r = min(row[i], M - 1);
    const float* rr = resid + (size_t)r * ep.ldr + cbase + cl;
    const float* gr = ep.mods ? ep.mods + (size_t)(ep.rows ? ep.rows[r] : 0) * ep.mstride + ep.goff + cbase + cl
                              : nullptr;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      rv[i][j] = rr[32 * j];
      gv[i][j] = gr ? gr[32 * j] : 1.0f;
    }
  }
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    if (row[i] >= M) continue;
    float* orow = out + (size_t)row[i] * ep.ldc + cbase + cl;
#pragma unroll
    for (int j = 0; j < NC; ++j) orow[32 * j] = rv[i][j] + gv[i][j] * (acc[i][j] + bv[j]);
  }
}

// Gated residual of a wave's (32 MI) x (32 NI) strip whose rows all read one
// modulation row (the wave's vote in gemm_epilogue): one gate per column and lane,
// and the residual rows in batches of 8 whose loads are issued one batch ahead of
// the stores, so the strip waits for memory about twice instead of 2 MI times.
template <int MI, int NI>
DIT_DEV void epi_gated_uniform(const Epi& ep, f32x16_t (&acc)[MI][NI], int M, int rbase, int cbase,
                               int lane, int mrow) {
  const int cl = lane & 31, rh = (lane >> 5) * 4;
  const float* __restrict__ resid = ep.resid;
  float* __restrict__ out = (float*)ep.out;
  float gv[NI], bv[NI];
  const float* gr = ep.mods ? ep.mods + (size_t)mrow * ep.mstride + ep.goff + cbase + cl : nullptr;
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    gv[j] = gr ? gr[32 * j] : 1.0f;
    bv[j] = ep.bias ? ep.bias[cbase + 32 * j + cl] : 0.0f;
  }
  constexpr int NB = 2 * MI;  // batches of 8 rows: (mi, half of the 16 values)
  auto row_of = [&](int b, int i) { return rbase + (b >> 1) * 32 + ((8 * (b & 1) + i) >> 2) * 8 + rh + (i & 3); };
  float rv[2][8][NI];
  auto load = [&](int b, float (&dst)[8][NI]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float* rr = resid + (size_t)min(row_of(b, i), M - 1) * ep.ldr + cbase + cl;
#pragma unroll
      for (int j = 0; j < NI; ++j) dst[i][j] = rr[32 * j];
    }
  };
  load(0, rv[0]);
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if (b + 1 < NB) load(b + 1, rv[(b + 1) & 1]);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = row_of(b, i);
      if (row >= M) continue;
      float* orow = out + (size_t)row * ep.ldc + cbase + cl;
#pragma unroll
      for (int j = 0; j < NI; ++j)
        orow[32 * j] = rv[b & 1][i][j] + gv[j] * (acc[b >> 1][j][8 * (b & 1) + i] + bv[j]);
    }
  }
}

// ---------------------------------------------------------------- bf16 MFMA ----
// 256x256x64 workgroup tile, 512 threads = 8 waves as 4 (M) x 2 (N); each wave
// owns a 64x128 strip (2x4 blocks of 32x32, 128 fp32 accumulators per lane).
// The next K tile is loaded into registers one full MFMA section ahead of its
// LDS store (the loads of tile k+2 are issued right after tile k+1 is stored),
// so global latency hides behind a whole tile of MFMAs.  A partial last N tile
// (N % 256 != 0, N % 32 == 0) clamps its B rows and masks its stores (per
// 128-column wave strip, and per 32-column block in the plain-store epilogue).
constexpr int GBM = 256, GBK = 64;
constexpr int GWM = 4, GWN = 2;                 // wave grid
constexpr int GTM = GBM / GWM;  // 64 rows per wave
constexpr int GMI = GTM / 32;
constexpr int kQkvNI = 4;  // the QKV epilogue's 128-column wave strips
constexpr int GNT = 64 * GWM * GWN;             // 512 threads
constexpr int GCPR = GBK / 8;                   // 16-byte chunks per tile row
constexpr int GAL = GBM * GCPR / GNT;
constexpr int kGroupM = 4;  // tile rows per rasterization group

// LDS element offset of 16-byte chunk `ch` of row `r` in a [rows][64] bf16
// tile.  The chunk index is XOR-ed with (r / 2) % 8: the 16 rows that one
// quarter-wave's ds_read_b128 touches then cover all 64 banks exactly once.
DIT_DEV int swz64(int r, int ch) { return r * GBK + ((ch ^ ((r >> 1) & 7)) << 3); }

// QKV epilogue of one wave's 64 x 128 strip, which covers whole heads (128
// columns = one head of 128 or two of 64; strips start on head boundaries).
// Per token and head ([MMH3] norm_rope_w; qk-norm before rotary as [ENC]
// rms_norm_heads): q and k are RMS-normalized with the shared [hd] gain,
// rotated pairwise by the token's angles, q is scaled by q_scale (the
// softmax's base-2 score scale) and both are written head-major; v goes out transposed
// per head (keys contiguous) for the attention kernel's second product.
// Rows are finished one at a time so that only the accumulators stay live.
template <int HD, int ROPE, int MI>
DIT_DEV void epi_qk_rows(const Epi& ep, f32x16_t (&acc)[MI][kQkvNI], int M, int rbase, int c0,
                         int which, int lane) {
  constexpr int P = HD / 2;
  const int cl = lane & 31, rh = (lane >> 5) * 4;
  const int ldn = ep.ldn;
  const float* g = which ? ep.kn : ep.qn;
  const float qs = which == 0 ? ep.q_scale : 1.0f;
  bf16_t* dst = (bf16_t*)(which ? ep.k : ep.q);
  const float2* cs = (const float2*)ep.cs;
  float gv[kQkvNI];
#pragma unroll
  for (int ni = 0; ni < kQkvNI; ++ni) gv[ni] = g ? g[(32 * ni + cl) & (HD - 1)] : 1.0f;
  const bool even = (cl & 1) == 0;
  // The rows' (cos, sin) pairs are fetched in batches of RB rows, one batch
  // ahead of the rows that use them, so that the strip waits for them about once
  // instead of once per row.  NCS pairs per row and lane: split-half 2 (hd 128:
  // pairs cl and cl + 32) or 1 (hd 64), interleaved one per 32-column block.
  constexpr int NCS = ROPE == 0 ? 0 : ROPE == 1 ? (HD == 128 ? 2 : 1) : kQkvNI;
  constexpr int NCA = NCS > 0 ? NCS : 1;
  constexpr int RB = NCS <= 2 ? 8 : 4;
  constexpr int BPM = 16 / RB, NB = MI * BPM;
  auto row_of = [&](int b, int i) {
    const int v = (b % BPM) * RB + i;
    return rbase + (b / BPM) * 32 + (v >> 2) * 8 + rh + (v & 3);
  };
  auto cs_index = [&](int c) {
    return ROPE == 1 ? (HD == 128 ? 32 * c + cl : cl) : ((32 * c + cl) & (HD - 1)) >> 1;
  };
  float2 csb[2][RB][NCA];
  auto load_cs = [&](int b, float2 (&d)[RB][NCA]) __attribute__((always_inline)) {
    if (NCS == 0) return;
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const float2* csr = cs + (size_t)min(row_of(b, i), M - 1) * P;
#pragma unroll
      for (int c = 0; c < NCS; ++c) d[i][c] = csr[cs_index(c)];
    }
  };
  load_cs(0, csb[0]);
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if (b + 1 < NB) load_cs(b + 1, csb[(b + 1) & 1]);
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int mi = b / BPM, v = (b % BPM) * RB + i;
      const int row = row_of(b, i);
      const float2* cr = csb[b & 1][i];
      float x[kQkvNI];
#pragma unroll
      for (int ni = 0; ni < kQkvNI; ++ni) x[ni] = acc[mi][ni][v];
      if (g) {
        // blocks 0..3 are one head (HD = 128) or two (HD = 64: 0-1 and 2-3); the
        // other 31 lanes of this half-wave hold the rest of the row's columns
        float s0 = (HD == 128) ? (x[0] * x[0] + x[1] * x[1]) + (x[2] * x[2] + x[3] * x[3])
                               : x[0] * x[0] + x[1] * x[1];
        float s1 = (HD == 128) ? 0.0f : x[2] * x[2] + x[3] * x[3];
        s0 = sum32(s0);
        if (HD != 128) s1 = sum32(s1);
        // v_rsq_f32 (about one ulp): the result is rounded to bf16
        const float i0 = __builtin_amdgcn_rsqf(s0 * (1.0f / HD) + ep.qk_eps);
        const float i1 = (HD == 128) ? i0 : __builtin_amdgcn_rsqf(s1 * (1.0f / HD) + ep.qk_eps);
#pragma unroll
        for (int ni = 0; ni < kQkvNI; ++ni) x[ni] *= ((HD == 128 || ni < 2) ? i0 : i1) * gv[ni];
      }
      if (ROPE == 1) {  // split-half: pair (d, d + P) is in this lane, blocks ni, ni + P/32
        if (HD == 128) {
#pragma unroll
          for (int ni = 0; ni < 2; ++ni) {
            const float2 c = cr[ni];
            const float a = x[ni], bb = x[ni + 2];
            x[ni] = a * c.x - bb * c.y;
            x[ni + 2] = a * c.y + bb * c.x;
          }
        } else {
          const float2 c = cr[0];
#pragma unroll
          for (int ni = 0; ni < kQkvNI; ni += 2) {
            const float a = x[ni], bb = x[ni + 1];
            x[ni] = a * c.x - bb * c.y;
            x[ni + 1] = a * c.y + bb * c.x;
          }
        }
      } else if (ROPE == 2) {  // interleaved: pair (2i, 2i + 1) is in lanes cl and cl ^ 1
#pragma unroll
        for (int ni = 0; ni < kQkvNI; ++ni) {
          const float oth = DIT_DPP(x[ni], 0xB1);  // lane ^ 1
          const float2 c = cr[ni];
          const float xe = even ? x[ni] : oth, xo = even ? oth : x[ni];
          x[ni] = even ? (xe * c.x - xo * c.y) : (xe * c.y + xo * c.x);
        }
      }
      if (row < ldn) {
        const bool valid = row < M;
#pragma unroll
        for (int ni = 0; ni < kQkvNI; ++ni) {
          const int col = c0 + 32 * ni + cl;
          const int h = col / HD, d = col - h * HD;
          dst[((size_t)h * ldn + row) * HD + d] = f2bf(valid ? x[ni] * qs : 0.0f);
        }
      }
    }
  }
}

template <int MI>
DIT_DEV void epi_qkv(const Epi& ep, f32x16_t (&acc)[MI][kQkvNI], int M, int rbase, int cbase,
                     int lane) {
  const int cl = lane & 31, rh = (lane >> 5) * 4;
  const int D = ep.ldc, ldn = ep.ldn;
  const int which = cbase / D;       // 0 q, 1 k, 2 v
  const int c0 = cbase - which * D;  // first column of the strip inside its q/k/v block
  if (ep.bias) {
#pragma unroll
    for (int ni = 0; ni < kQkvNI; ++ni) {
      const float b = ep.bias[cbase + 32 * ni + cl];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[mi][ni][v] += b;
    }
  }
  if (which == 2) {
    // v^T [H, hd, ldn]: a lane holds 4 consecutive rows of one column per (mi, ni, v/4)
    bf16_t* vt = (bf16_t*)ep.vt;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int vq = 0; vq < 4; ++vq) {
        const int row0 = rbase + mi * 32 + vq * 8 + rh;
        if (row0 >= ldn) continue;  // ldn is a multiple of 128: all four rows in or out
#pragma unroll
        for (int ni = 0; ni < kQkvNI; ++ni) {
          const int col = c0 + 32 * ni + cl;  // h * hd + d
          float e[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) e[j] = (row0 + j < M) ? acc[mi][ni][vq * 4 + j] : 0.0f;
          *(uint2*)(vt + (size_t)col * ldn + row0) = make_uint2(pack2bf(e[0], e[1]), pack2bf(e[2], e[3]));
        }
      }
    return;
  }
  switch (ep.hd * 4 + ep.rope) {
    case 128 * 4 + 0: epi_qk_rows<128, 0, MI>(ep, acc, M, rbase, c0, which, lane); break;
    case 128 * 4 + 1: epi_qk_rows<128, 1, MI>(ep, acc, M, rbase, c0, which, lane); break;
    case 128 * 4 + 2: epi_qk_rows<128, 2, MI>(ep, acc, M, rbase, c0, which, lane); break;
    case 64 * 4 + 0: epi_qk_rows<64, 0, MI>(ep, acc, M, rbase, c0, which, lane); break;
    case 64 * 4 + 1: epi_qk_rows<64, 1, MI>(ep, acc, M, rbase, c0, which, lane); break;
    default: epi_qk_rows<64, 2, MI>(ep, acc, M, rbase, c0, which, lane); break;
  }
}

// Epilogue of one wave's (32 MI) x (32 NI) accumulator strip whose first row is
// rbase and first column cbase (< N).  C layout of a 32x32 block: lane holds column
// (lane & 31) and rows 8*(v/4) + 4*(lane/32) + v%4 for v = 0..15.
template <int EPI, typename OutT, int MI, int NI>
DIT_DEV void gemm_epilogue(const Epi& ep, f32x16_t (&acc)[MI][NI], int M, int N, int rbase,
                           int cbase, int lane) {
  const int cl = lane & 31, rh = (lane >> 5) * 4;
  if constexpr (EPI == EPI_QKV) {
    epi_qkv<MI>(ep, acc, M, rbase, cbase, lane);
    return;
  }
  if constexpr (EPI == EPI_GATED_RES) {
    // the strip's 32 MI rows, one per lane: do they share one modulation row?
    int mrow = 0;
    bool uniform = true;
    if (ep.mods && ep.rows) {
      mrow = ep.rows[min(rbase, M - 1)];
      const int own = ep.rows[min(rbase + (lane & (32 * MI - 1)), M - 1)];
      uniform = __all(own == mrow);
    }
    if (uniform) {
      epi_gated_uniform<MI, NI>(ep, acc, M, rbase, cbase, lane, mrow);
      return;
    }
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int vh = 0; vh < 2; ++vh) {
        int rows8[8];
        float a8[8][NI];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int v = vh * 8 + i;
          rows8[i] = rbase + mi * 32 + (v >> 2) * 8 + rh + (v & 3);
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) a8[i][ni] = acc[mi][ni][v];
        }
        epi_gated_rows<8, NI>(ep, rows8, M, cbase, cl, a8);
      }
    return;
  }
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = rbase + mi * 32 + (v >> 2) * 8 + rh + (v & 3);
      if (row >= M) continue;
      if (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int ni = 0; ni < NI; ni += 2)
          epi_swiglu<OutT>(ep, row, (cbase + ni * 32) / 2 + cl, acc[mi][ni][v], acc[mi][ni + 1][v]);
      } else {
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          if (cbase + ni * 32 < N)  // N % 32 == 0: whole 32-column blocks in or out
            epi_one<EPI, OutT>(ep, row, cbase + ni * 32 + cl, acc[mi][ni][v]);
      }
    }
  }
}

// Tile L of the raster: groups of kGroupM tile rows, row index fastest.
DIT_DEV void tile_of(int L, int ntm, int ntn, int& tm, int& tn) {
  const int gsz = kGroupM * ntn, g = L / gsz, gr = L - g * gsz;
  const int gm = min(kGroupM, ntm - g * kGroupM);
  tm = g * kGroupM + gr % gm;
  tn = gr / gm;
}

// Split-K tail: tiles [F, total) of the raster, the ones a last partial round over
// the CUs would leave alone on a mostly idle chip, are each computed as S
// workgroups over consecutive K ranges; each writes its fp32 accumulators, in
// register order, to its slot of ep.split and the fixup kernel sums the S slots in
// order (deterministic) and applies the epilogue.
template <int NI>
constexpr int split_slot_floats() { return GMI * NI * 16 * 64 * (GNT / 64); }

template <int EPI, typename OutT, int NI>
__global__ __launch_bounds__(GNT) void k_gemm_bf16(const bf16_t* __restrict__ A, int lda,
                                                   const bf16_t* __restrict__ B, int ldb, int M,
                                                   int N, int K, int F, int S, Epi ep) {
  // NI 32-column blocks per wave: the tile is 256 x 64*NI (NI = 4, or 3 for widths that
  // are a multiple of 192 but not of 256)
  constexpr int GNI = NI, GTN = 32 * NI, GBN = GWN * GTN, GBL = GBN * GCPR / GNT;
  static_assert(GBN * GCPR % GNT == 0, "whole 16-byte chunks per thread");
  static_assert(EPI != EPI_QKV || NI == 4, "the QKV epilogue takes whole 128-column heads");
  static_assert(EPI != EPI_SWIGLU || NI % 2 == 0, "SwiGLU pairs 32-column blocks");
  __shared__ __attribute__((aligned(16))) bf16_t smem[2 * (GBM + GBN) * GBK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / GWN, wn = wave % GWN;
  // Tile order.  Workgroup i is dispatched to XCD i % 8 and each XCD has its
  // own L2, so every XCD gets a contiguous chunk of the tile sequence, and the
  // sequence runs through groups of kGroupM tile rows with the row index
  // fastest: the workgroups resident on one XCD then share both A row panels
  // and B column panels in its L2.  Workgroups from F on (F a multiple of 8)
  // are the split tail, S per tile.
  const int ntn = (N + GBN - 1) / GBN, ntm = (M + GBM - 1) / GBM;
  const int total = ntn * ntm;
  int L, part = -1;
  if (EPI == EPI_QKV || (int)blockIdx.x < F) {  // QKV launches never split
    L = (blockIdx.x % 8) * (F / 8) + blockIdx.x / 8;
    if (L >= total) return;
  } else {
    const int j = blockIdx.x - F;
    L = F + j / S;
    part = j;
    const int nkt = K / GBK, p = j % S, kb = nkt * p / S, ke = nkt * (p + 1) / S;
    A += (size_t)kb * GBK;
    B += (size_t)kb * GBK;
    K = (ke - kb) * GBK;
  }
  int tm, tn;
  tile_of(L, ntm, ntn, tm, tn);
  const int m0 = tm * GBM, n0 = tn * GBN;

  u32x4_t ra[GAL], rb[GBL];
#define GEMM_GLOAD(k0)                                                                   \
  do {                                                                                   \
    _Pragma("unroll") for (int i = 0; i < GAL; ++i) {                                    \
      const int c_ = tid + GNT * i, r_ = c_ / GCPR, ch_ = c_ % GCPR;                     \
      ra[i] = *(const u32x4_t*)(A + (size_t)min(m0 + r_, M - 1) * lda + (k0) + ch_ * 8); \
    }                                                                                    \
    _Pragma("unroll") for (int i = 0; i < GBL; ++i) {                                    \
      const int c_ = tid + GNT * i, r_ = c_ / GCPR, ch_ = c_ % GCPR;                     \
      rb[i] = *(const u32x4_t*)(B + (size_t)min(n0 + r_, N - 1) * ldb + (k0) + ch_ * 8); \
    }                                                                                    \
  } while (0)
#define GEMM_SSTORE(buf)                                                                 \
  do {                                                                                   \
    bf16_t* As_ = smem + (buf) * (GBM + GBN) * GBK;                                      \
    bf16_t* Bs_ = As_ + GBM * GBK;                                                       \
    _Pragma("unroll") for (int i = 0; i < GAL; ++i) {                                    \
      const int c_ = tid + GNT * i;                                                      \
      *(u32x4_t*)(As_ + swz64(c_ / GCPR, c_ % GCPR)) = ra[i];                            \
    }                                                                                    \
    _Pragma("unroll") for (int i = 0; i < GBL; ++i) {                                    \
      const int c_ = tid + GNT * i;                                                      \
      *(u32x4_t*)(Bs_ + swz64(c_ / GCPR, c_ % GCPR)) = rb[i];                            \
    }                                                                                    \
  } while (0)

  f32x16_t acc[GMI][GNI];
#pragma unroll
  for (int i = 0; i < GMI; ++i)
#pragma unroll
    for (int j = 0; j < GNI; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int nk = K / GBK;
  GEMM_GLOAD(0);
  GEMM_SSTORE(0);
  GEMM_GLOAD(min(1, nk - 1) * GBK);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const bf16_t* As = smem + (kt & 1) * (GBM + GBN) * GBK;
    const bf16_t* Bs = As + GBM * GBK;
#pragma unroll
    for (int s = 0; s < GBK / 16; ++s) {
      const int ch = 2 * s + (lane >> 5);
      bf16x8_t a[GMI], b[GNI];
#pragma unroll
      for (int mi = 0; mi < GMI; ++mi)
        a[mi] = *(const bf16x8_t*)(As + swz64(wm * GTM + mi * 32 + (lane & 31), ch));
#pragma unroll
      for (int ni = 0; ni < GNI; ++ni)
        b[ni] = *(const bf16x8_t*)(Bs + swz64(wn * GTN + ni * 32 + (lane & 31), ch));
#pragma unroll
      for (int mi = 0; mi < GMI; ++mi)
#pragma unroll
        for (int ni = 0; ni < GNI; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
    }
    // Unconditional: on the last two iterations these re-load the last tile
    // and fill the buffer nobody reads again, which keeps the staging
    // registers out of control flow (they stay in VGPRs).
    GEMM_SSTORE((kt + 1) & 1);
    GEMM_GLOAD(min(kt + 2, nk - 1) * GBK);
    // Issue order of the iteration: the first step's fragment reads, then
    // every MFMA of steps 0..2 followed by one fragment read of the next step,
    // and the last step's MFMAs each followed by one LDS store and one global
    // load of the staged tile, so neither burst leaves the matrix pipe idle.
    {
      constexpr int NR = GMI + GNI, NM = GMI * GNI, NS = GBK / 16, NL = GAL + GBL;
      static_assert(NM >= NR, "schedule pattern");
      __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);  // ds_read
#pragma unroll
      for (int st = 0; st < NS - 1; ++st) {
#pragma unroll
        for (int i = 0; i < NR; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // ds_read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, NM - NR, 0);
      }
      constexpr int NP = NL < NM ? NL : NM;  // staged chunks paired with an MFMA
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // ds_write
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global load
      }
      if (NM > NP) __builtin_amdgcn_sched_group_barrier(0x008, NM - NP, 0);
      if (NL > NP) {
        __builtin_amdgcn_sched_group_barrier(0x200, NL - NP, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, NL - NP, 0);
      }
    }
    __syncthreads();
  }
#undef GEMM_GLOAD
#undef GEMM_SSTORE

  // a split-tail workgroup: accumulators to its slot, in register order (not for
  // QKV: a second reader of the accumulators beside its epilogue makes the
  // register allocation spill; its launches never split)
  if constexpr (EPI != EPI_QKV) {
    if (part >= 0) {
      f32x4_t* dst = (f32x4_t*)(ep.split + (size_t)part * split_slot_floats<NI>()) +
                     (size_t)wave * GMI * GNI * 4 * 64 + lane;
#pragma unroll
      for (int mi = 0; mi < GMI; ++mi)
#pragma unroll
        for (int ni = 0; ni < GNI; ++ni)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            f32x4_t v4 = {acc[mi][ni][4 * q], acc[mi][ni][4 * q + 1], acc[mi][ni][4 * q + 2],
                          acc[mi][ni][4 * q + 3]};
            dst[((mi * GNI + ni) * 4 + q) * 64] = v4;
          }
      return;
    }
  }
  const int cbase = n0 + wn * GTN;
  if (cbase >= N) return;  // the masked half of a partial last N tile
  gemm_epilogue<EPI, OutT, GMI, GNI>(ep, acc, M, N, m0 + wm * GTM, cbase, lane);
}

// The split tail's second half: one wave per workgroup, workgroup 8 t + w sums wave
// w's accumulators of tile F + t over the S slots in slot order and applies the
// epilogue the unsplit kernel would have (one wave each: the reads and the epilogue
// spread over eight times as many CUs as the tail has tiles).
template <int EPI, typename OutT, int NI>
__global__ __launch_bounds__(64) void k_gemm_fixup(int M, int N, int F, int S, Epi ep) {
  constexpr int GNI = NI, GTN = 32 * NI, GBN = GWN * GTN;
  const int lane = threadIdx.x, t = blockIdx.x >> 3, wave = blockIdx.x & 7;
  const int wm = wave / GWN, wn = wave % GWN;
  const int ntn = (N + GBN - 1) / GBN, ntm = (M + GBM - 1) / GBM;
  int tm, tn;
  tile_of(F + t, ntm, ntn, tm, tn);
  const int m0 = tm * GBM, n0 = tn * GBN;
  const int cbase = n0 + wn * GTN;
  if (cbase >= N) return;
  f32x16_t acc[GMI][GNI];
  for (int p = 0; p < S; ++p) {
    const f32x4_t* src = (const f32x4_t*)(ep.split + (size_t)(t * S + p) * split_slot_floats<NI>()) +
                         (size_t)wave * GMI * GNI * 4 * 64 + lane;
#pragma unroll
    for (int mi = 0; mi < GMI; ++mi)
#pragma unroll
      for (int ni = 0; ni < GNI; ++ni)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4_t v4 = src[((mi * GNI + ni) * 4 + q) * 64];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[mi][ni][4 * q + e] = p ? acc[mi][ni][4 * q + e] + v4[e] : v4[e];
        }
  }
  gemm_epilogue<EPI, OutT, GMI, GNI>(ep, acc, M, N, m0 + wm * GTM, cbase, lane);
}

// ---------------------------------------------------------------- fp32 FMA ----
template <int EPI, typename OutT>
__global__ __launch_bounds__(256) void k_gemm_f32(const float* __restrict__ A, int lda,
                                                  const float* __restrict__ B, int ldb, int M,
                                                  int N, int K, Epi ep) {
  __shared__ float As[16][68], Bs[16][68];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int ntn = N / 64;
  const int tm = blockIdx.x / ntn, tn = blockIdx.x - tm * ntn;
  const int m0 = tm * 64, n0 = tn * 64;
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    int ar = m0 + lr;
    float4 av = make_float4(0.f, 0.f, 0.f, 0.f);
    if (ar < M) av = *(const float4*)(A + (size_t)ar * lda + k0 + lk);
    float4 bv = *(const float4*)(B + (size_t)(n0 + lr) * ldb + k0 + lk);
    As[lk + 0][lr] = av.x; As[lk + 1][lr] = av.y; As[lk + 2][lr] = av.z; As[lk + 3][lr] = av.w;
    Bs[lk + 0][lr] = bv.x; Bs[lk + 1][lr] = bv.y; Bs[lk + 2][lr] = bv.z; Bs[lk + 3][lr] = bv.w;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + ty + 16 * i;
    if (row >= M) continue;
    if (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int j = 0; j < 2; ++j) epi_swiglu<OutT>(ep, row, n0 / 2 + tx + 16 * j, acc[i][j], acc[i][j + 2]);
    } else if (EPI == EPI_GATED_RES) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + tx + 16 * j;
        float v = acc[i][j] + (ep.bias ? ep.bias[col] : 0.0f);
        float gate = ep.mods ? ep.mods[(size_t)(ep.rows ? ep.rows[row] : 0) * ep.mstride + ep.goff + col] : 1.0f;
        ((float*)ep.out)[(size_t)row * ep.ldc + col] = ep.resid[(size_t)row * ep.ldr + col] + gate * v;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) epi_one<EPI, OutT>(ep, row, n0 + tx + 16 * j, acc[i][j]);
    }
  }
}

// Launch plan of a bf16 GEMM: tile width, and the split-K tail if it pays.
struct GemmPlan {
  bool w192 = false;
  int F = 0, S = 1, tail = 0, grid = 0;
};

static GemmPlan plan_gemm(int epi, int M, int N, int K, bool can_split) {
  GemmPlan P;
  const int cus = device_cus(), tm = (M + GBM - 1) / GBM, nk = K / GBK;
  const int tiles4 = tm * ((N + 255) / 256);
  // Candidate costs in units of one 256 x 256 tile's time, per CU.  Plain 256-wide
  // tiles: whole rounds over the CUs.
  double best = (tiles4 + cus - 1) / cus;
  // 192-wide tiles where they divide N and 256-wide ones do not (N = 2688: 14 full
  // tiles per row instead of 10.5): a 256 x 192 tile takes about 0.86 of a 256 x 256
  // one (measured at N = 2688).
  if ((epi == EPI_GATED_RES || epi == EPI_STORE) && N % 256 != 0 && N % 192 == 0) {
    const double c3 = 0.86 * ((tm * (N / 192) + cus - 1) / cus);
    if (c3 < best) {
      best = c3;
      P.w192 = true;
    }
  }
  // Split-K tail: the tiles beyond the last whole round over the CUs, when they fill
  // at most half of them, each become S >= 2 workgroups over K ranges (at most
  // kGemmSplitWgs in all, at least two K tiles each): full rounds + 1/S, plus the
  // partial stores and the fixup pass (measured at N = 2688: about 0.2 of a tile
  // plus the time of 17 K steps).
  if (can_split && cus % 8 == 0) {
    const int full = tiles4 / cus * cus, tail = tiles4 - full;
    const int S = tail ? min(min(cus, kGemmSplitWgs) / tail, min(4, nk / 2)) : 1;
    if (tail && S >= 2) {
      const double cs = full / cus + 1.0 / S + 0.2 + 17.0 / nk;
      if (cs < best) {
        P.w192 = false;
        P.F = full;
        P.S = S;
        P.tail = tail;
        P.grid = full + tail * S;
        return P;
      }
    }
  }
  const int tiles = P.w192 ? tm * (N / 192) : tiles4;
  P.F = P.grid = (tiles + 7) / 8 * 8;  // a whole number of rounds over the 8 XCDs
  return P;
}

template <int EPI, typename OutT, int NI>
static void launch_bf16(const GemmPlan& P, const bf16_t* A, int lda, const bf16_t* B, int ldb,
                        int M, int N, int K, const Epi& ep, hipStream_t s) {
  k_gemm_bf16<EPI, OutT, NI><<<P.grid, GNT, 0, s>>>(A, lda, B, ldb, M, N, K, P.F, P.S, ep);
  if constexpr (EPI != EPI_QKV)
    if (P.tail) k_gemm_fixup<EPI, OutT, NI><<<P.tail * (GNT / 64), 64, 0, s>>>(M, N, P.F, P.S, ep);
}

template <int EPI>
static hipError_t launch_gemm(int dtype, bool out_bf16, const void* A, int lda, const void* B,
                              int ldb, int M, int N, int K, const Epi& ep, hipStream_t s) {
  if (dtype == BF16) {
    const GemmPlan P = plan_gemm(EPI, M, N, K, EPI != EPI_QKV && ep.split != nullptr);
    const bf16_t *Ab = (const bf16_t*)A, *Bb = (const bf16_t*)B;
    if constexpr (EPI == EPI_QKV) {
      launch_bf16<EPI, bf16_t, 4>(P, Ab, lda, Bb, ldb, M, N, K, ep, s);
    } else if constexpr (EPI == EPI_GATED_RES) {
      if (P.w192)
        launch_bf16<EPI, bf16_t, 3>(P, Ab, lda, Bb, ldb, M, N, K, ep, s);
      else
        launch_bf16<EPI, bf16_t, 4>(P, Ab, lda, Bb, ldb, M, N, K, ep, s);
    } else if constexpr (EPI == EPI_STORE) {
      if (out_bf16 && P.w192) launch_bf16<EPI, bf16_t, 3>(P, Ab, lda, Bb, ldb, M, N, K, ep, s);
      else if (out_bf16) launch_bf16<EPI, bf16_t, 4>(P, Ab, lda, Bb, ldb, M, N, K, ep, s);
      else if (P.w192) launch_bf16<EPI, float, 3>(P, Ab, lda, Bb, ldb, M, N, K, ep, s);
      else launch_bf16<EPI, float, 4>(P, Ab, lda, Bb, ldb, M, N, K, ep, s);
    } else {
      if (out_bf16)
        launch_bf16<EPI, bf16_t, 4>(P, Ab, lda, Bb, ldb, M, N, K, ep, s);
      else
        launch_bf16<EPI, float, 4>(P, Ab, lda, Bb, ldb, M, N, K, ep, s);
    }
  } else {
    if constexpr (EPI == EPI_QKV) {
      return hipErrorInvalidValue;
    } else {
      dim3 grid(((M + 63) / 64) * (N / 64));
      k_gemm_f32<EPI, float><<<grid, 256, 0, s>>>((const float*)A, lda, (const float*)B, ldb, M,
                                                   N, K, ep);
    }
  }
  return hipGetLastError();
}

hipError_t gemm(int dtype, int epi, bool out_bf16, const void* A, int lda, const void* B, int ldb,
                int M, int N, int K, const Epi& ep, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  switch (epi) {
    case EPI_STORE: return launch_gemm<EPI_STORE>(dtype, out_bf16, A, lda, B, ldb, M, N, K, ep, s);
    case EPI_GATED_RES: return launch_gemm<EPI_GATED_RES>(dtype, out_bf16, A, lda, B, ldb, M, N, K, ep, s);
    case EPI_SWIGLU: return launch_gemm<EPI_SWIGLU>(dtype, out_bf16, A, lda, B, ldb, M, N, K, ep, s);
    case EPI_GELU: return launch_gemm<EPI_GELU>(dtype, out_bf16, A, lda, B, ldb, M, N, K, ep, s);
    case EPI_QKV:
      if (dtype != BF16) return hipErrorInvalidValue;
      return launch_gemm<EPI_QKV>(dtype, true, A, lda, B, ldb, M, N, K, ep, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace dit
