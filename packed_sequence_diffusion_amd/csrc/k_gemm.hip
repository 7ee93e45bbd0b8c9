// GEMMs of the block, C[M, N] = A[M, K] * B[N, K]^T (both operands K-contiguous,
// weights stored [out, in]), with the epilogues fused into the store:
// plain/bias store, gated residual ([MMH3] residual), SwiGLU pairing ([MMH3]
// ffn_tail) and bias + GELU-tanh ([SIGLIP] GeluBiasOp).
//
// bf16 path: v_mfma_f32_32x32x16_bf16 on LDS-staged 256x128x64 tiles; four
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
    Elt<OutT>::st((OutT*)ep.out + (size_t)row * ep.ldc + col, v);
  } else if (EPI == EPI_GATED_RES) {
    if (ep.bias) v += ep.bias[col];
    float gate = 1.0f;
    if (ep.mods) gate = ep.mods[(size_t)(ep.rows ? ep.rows[row] : 0) * ep.mstride + ep.goff + col];
    float* o = (float*)ep.out + (size_t)row * ep.ldc + col;
    *o = ep.resid[(size_t)row * ep.ldr + col] + gate * v;
  } else if (EPI == EPI_GELU) {
    if (ep.bias) v += ep.bias[col];
    Elt<OutT>::st((OutT*)ep.out + (size_t)row * ep.ldc + col, gelu_tanh_f(v));
  }
}

template <typename OutT>
DIT_DEV void epi_swiglu(const Epi& ep, int row, int ocol, float g, float u) {
  Elt<OutT>::st((OutT*)ep.out + (size_t)row * ep.ldc + ocol, silu_f(g) * u);
}

// ---------------------------------------------------------------- bf16 MFMA ----
constexpr int GBM = 256, GBN = 128, GBK = 64;

// LDS element offset of 16-byte chunk `ch` (0..7) of row `r` in a [rows][64]
// bf16 tile; the chunk index is XOR-swizzled with the row so that 8
// consecutive rows reading the same logical chunk hit 8 different bank groups.
DIT_DEV int swz64(int r, int ch) { return r * GBK + ((ch ^ (r & 7)) << 3); }

template <int EPI, typename OutT>
__global__ __launch_bounds__(256) void k_gemm_bf16(const bf16_t* __restrict__ A, int lda,
                                                   const bf16_t* __restrict__ B, int ldb, int M,
                                                   int N, int K, Epi ep) {
  __shared__ __attribute__((aligned(16))) bf16_t smem[2 * (GBM + GBN) * GBK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ntn = N / GBN;
  const int tm = blockIdx.x / ntn, tn = blockIdx.x - tm * ntn;
  const int m0 = tm * GBM, n0 = tn * GBN;
  const int lrow = tid >> 3, lch = tid & 7;

  uint4 ra[8], rb[4];
#define GEMM_GLOAD(k0)                                                              \
  do {                                                                              \
    _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                 \
      int gr = min(m0 + lrow + 32 * i, M - 1);                                      \
      ra[i] = *(const uint4*)(A + (size_t)gr * lda + (k0) + lch * 8);               \
    }                                                                               \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) rb[i] =                           \
        *(const uint4*)(B + (size_t)(n0 + lrow + 32 * i) * ldb + (k0) + lch * 8);   \
  } while (0)
#define GEMM_SSTORE(buf)                                                            \
  do {                                                                              \
    bf16_t* As_ = smem + (buf) * (GBM + GBN) * GBK;                                 \
    bf16_t* Bs_ = As_ + GBM * GBK;                                                  \
    _Pragma("unroll") for (int i = 0; i < 8; ++i)                                   \
        *(uint4*)(As_ + swz64(lrow + 32 * i, lch)) = ra[i];                         \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                   \
        *(uint4*)(Bs_ + swz64(lrow + 32 * i, lch)) = rb[i];                         \
  } while (0)

  f32x16_t acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int nk = K / GBK;
  GEMM_GLOAD(0);
  GEMM_SSTORE(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) GEMM_GLOAD((kt + 1) * GBK);
    const bf16_t* As = smem + buf * (GBM + GBN) * GBK;
    const bf16_t* Bs = As + GBM * GBK;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int ch = 2 * s + (lane >> 5);
      bf16x8_t a[2], b[4];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
        a[mi] = *(const bf16x8_t*)(As + swz64(wave * 64 + mi * 32 + (lane & 31), ch));
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
        b[ni] = *(const bf16x8_t*)(Bs + swz64(ni * 32 + (lane & 31), ch));
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
    }
    if (kt + 1 < nk) GEMM_SSTORE(buf ^ 1);
    __syncthreads();
  }

  // C layout of a 32x32 block: lane holds column (lane & 31) and rows
  // 8*(v/4) + 4*(lane/32) + v%4 for v = 0..15.
  const int cl = lane & 31, rh = (lane >> 5) * 4;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = m0 + wave * 64 + mi * 32 + (v >> 2) * 8 + rh + (v & 3);
      if (row >= M) continue;
      if (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int ni = 0; ni < 4; ni += 2)
          epi_swiglu<OutT>(ep, row, (n0 + ni * 32) / 2 + cl, acc[mi][ni][v], acc[mi][ni + 1][v]);
      } else {
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) epi_one<EPI, OutT>(ep, row, n0 + ni * 32 + cl, acc[mi][ni][v]);
      }
    }
  }
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
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) epi_one<EPI, OutT>(ep, row, n0 + tx + 16 * j, acc[i][j]);
    }
  }
}

template <int EPI>
static hipError_t launch_gemm(int dtype, bool out_bf16, const void* A, int lda, const void* B,
                              int ldb, int M, int N, int K, const Epi& ep, hipStream_t s) {
  if (dtype == BF16) {
    dim3 grid(((M + GBM - 1) / GBM) * (N / GBN));
    if (out_bf16 || EPI == EPI_GATED_RES)
      k_gemm_bf16<EPI, bf16_t><<<grid, 256, 0, s>>>((const bf16_t*)A, lda, (const bf16_t*)B, ldb,
                                                     M, N, K, ep);
    else
      k_gemm_bf16<EPI, float><<<grid, 256, 0, s>>>((const bf16_t*)A, lda, (const bf16_t*)B, ldb,
                                                    M, N, K, ep);
  } else {
    dim3 grid(((M + 63) / 64) * (N / 64));
    k_gemm_f32<EPI, float><<<grid, 256, 0, s>>>((const float*)A, lda, (const float*)B, ldb, M, N,
                                                 K, ep);
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
  }
  return hipErrorInvalidValue;
}

}  // namespace dit
