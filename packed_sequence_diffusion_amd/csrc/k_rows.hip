// Bandwidth-bound kernels of the block: adaLN interpolation, pre-norm +
// modulate, sandwich residual, RoPE table, qk-norm/RoPE head split, weight prep.
//
// Citation tags: [MMH3] docs.rs source page of cortiq-engine 0.5.72,
// src/mmh3.rs; [SIGLIP] ffai-argus 0.7.0, src/siglip.rs; [ZIMG] ollama's
// zimage transformer.go.
#include "dev_common.h"
#include "dit_kernels.h"

namespace dit {

// ------------------------------------------------------------------------------
// adaLN: mods[j] = bias[j] + sum_k basis[j, k] * c_s[k], s = j / per_slot,
// c_s = table[i0_s] + f_s * (table[i0_s + 1] - table[i0_s])   ([MMH3] Adaln::eval)
// One thread per flat element j; the basis row is read as rank/4 float4.
// ------------------------------------------------------------------------------
template <int RANK4>
__global__ __launch_bounds__(256) void k_adaln_interp(const float* __restrict__ basis,
                                                      const float* __restrict__ bias,
                                                      const float* __restrict__ table,
                                                      int rank, int per_slot, int total,
                                                      SlotCoords sc, float* __restrict__ mods) {
  int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= total) return;
  int s = j / per_slot;
  const float* t0 = table + (size_t)sc.i0[s] * rank;
  const float* t1 = t0 + rank;
  float f = sc.f[s];
  float acc = bias ? bias[j] : 0.0f;
  if (RANK4 > 0) {
    const float4* b4 = (const float4*)(basis + (size_t)j * rank);
    const float4* a4 = (const float4*)t0;
    const float4* c4 = (const float4*)t1;
#pragma unroll
    for (int q = 0; q < RANK4; ++q) {
      float4 b = b4[q], a = a4[q], c = c4[q];
      acc += b.x * (a.x + f * (c.x - a.x));
      acc += b.y * (a.y + f * (c.y - a.y));
      acc += b.z * (a.z + f * (c.z - a.z));
      acc += b.w * (a.w + f * (c.w - a.w));
    }
  } else {
    const float* b = basis + (size_t)j * rank;
    for (int k = 0; k < rank; ++k) acc += b[k] * (t0[k] + f * (t1[k] - t0[k]));
  }
  mods[j] = acc;
}

hipError_t adaln_interp(const float* basis, const float* bias, const float* table, int rank,
                        int per_slot, int slots, const SlotCoords& sc, float* mods,
                        hipStream_t s) {
  int total = per_slot * slots;
  dim3 grid((total + 255) / 256);
  if (rank == 24)
    k_adaln_interp<6><<<grid, 256, 0, s>>>(basis, bias, table, rank, per_slot, total, sc, mods);
  else
    k_adaln_interp<0><<<grid, 256, 0, s>>>(basis, bias, table, rank, per_slot, total, sc, mods);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------
// Z-Image timestep embedding and adaLN ([ZIMG] TimestepEmbedder.Forward and
// TransformerBlock.Forward): e = [cos(t f_i) | sin(t f_i)], f_i =
// exp(-ln(10000) i / half); h = silu(W1 e + b1); temb = W2 h + b2;
// mods = Wa temb + ba.  The sinusoid is evaluated once, in fp64; each dense
// layer gives one wave to each output, the lanes striding over the inputs so
// that a wave reads its weight row contiguously.
// ------------------------------------------------------------------------------
__global__ void k_temb_sin(double t, int half, float* __restrict__ e) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= half) return;
  double a = t * exp(-log(10000.0) * (double)i / (double)half);
  e[i] = (float)cos(a);
  e[half + i] = (float)sin(a);
}

template <bool SILU>
__global__ __launch_bounds__(256) void k_dense(const float* __restrict__ x, int in, int out,
                                               const float* __restrict__ w,
                                               const float* __restrict__ b,
                                               float* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int o = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (o >= out) return;
  const float* wr = w + (size_t)o * in;
  float acc = 0.0f;
  for (int i = lane; i < in; i += 64) acc += wr[i] * x[i];
  acc = wave_sum(acc) + (b ? b[o] : 0.0f);
  if (lane == 0) y[o] = SILU ? silu_f(acc) : acc;
}

hipError_t temb_mods(double t_scaled, int freq, int hidden, int out_dim, const float* w1,
                     const float* b1, const float* w2, const float* b2, const float* wa,
                     const float* ba, float* scratch, float* mods, hipStream_t s, bool silu_temb) {
  // scratch: h [hidden] then one [freq] slot that holds the sinusoid e until
  // the first layer has read it, then temb.
  float* h = scratch;
  float* et = scratch + hidden;
  const int half = freq / 2;
  k_temb_sin<<<(half + 127) / 128, 128, 0, s>>>(t_scaled, half, et);
  k_dense<true><<<(hidden + 3) / 4, 256, 0, s>>>(et, freq, hidden, w1, b1, h);
  // the final layer's adaLN reads silu(temb) ([ZIMG] FinalLayer.Forward)
  if (silu_temb)
    k_dense<true><<<(freq + 3) / 4, 256, 0, s>>>(h, hidden, freq, w2, b2, et);
  else
    k_dense<false><<<(freq + 3) / 4, 256, 0, s>>>(h, hidden, freq, w2, b2, et);
  k_dense<false><<<(out_dim + 3) / 4, 256, 0, s>>>(et, freq, out_dim, wa, ba, mods);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------
// Pre-norm + modulate, one wave per token row, the row held in registers
// ([MMH3] norm_rows + modulate; [SIGLIP] layer_norm; [ZIMG] RMSNorm * (1 + scale)).
//   RMS:   y = x / sqrt(mean(x^2) + eps) * g
//   LAYER: y = (x - mean) / sqrt(var + eps) * g + beta   (two passes in registers)
//   then y * (1 + mods[r, scale]) (+ mods[r, shift]);  y = (x - mean) * inv * G + B
// with the multiplier G = g (1 + scale) and the additive term B = beta (1 + scale)
// + shift.  A block is four consecutive rows.  When they share their segment row
// (all but a few blocks of a packing), the block builds G and B once in LDS
// (2 D floats) before its rows are read: fetching the three D-vectors from L2
// for every row costs the kernel about a fifth of its time at D = 2688.  A block
// whose rows differ reads them per chunk from L2.  Rows are read and outputs
// written once, with non-temporal accesses.  NCH = float4 chunks per lane
// (D <= 256 * NCH).
// ------------------------------------------------------------------------------
constexpr int kMaxChunks = 16;  // D <= 4096: 1024 float4 per row, 16 per lane
constexpr int kNormRows = 4;    // rows (waves) per block

template <int NORM, int MOD, int NCH, typename OutT>
__global__ __launch_bounds__(64 * kNormRows) void k_norm_mod(
    const float* __restrict__ x, int n, int D, const float* __restrict__ g,
    const float* __restrict__ beta, float eps, const float* __restrict__ mods, int mstride,
    const int* __restrict__ rows, int shift_off, int scale_off, OutT* __restrict__ y) {
  extern __shared__ float4 gb_lds[];  // [0, nc): G, [nc, 2 nc): B
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int row0 = blockIdx.x * kNormRows;
  const int row = row0 + (t >> 6);
  const int nc = D >> 2;
  const bool per_row = MOD != MOD_NONE && rows != nullptr;
  // G and B of modulation row mr, chunk i (0 <= i < nc)
  auto gb = [&](int mr, int i, float4& G, float4& B) {
    G = ((const float4*)g)[i];
    B = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (NORM == NORM_LAYER) B = ((const float4*)beta)[i];
    if (MOD != MOD_NONE) {
      const float* mrow = mods + (size_t)mr * mstride;
      const float4 sc = ((const float4*)(mrow + scale_off))[i];
      G = make_float4(G.x * (1.0f + sc.x), G.y * (1.0f + sc.y), G.z * (1.0f + sc.z),
                      G.w * (1.0f + sc.w));
      if (NORM == NORM_LAYER)
        B = make_float4(B.x * (1.0f + sc.x), B.y * (1.0f + sc.y), B.z * (1.0f + sc.z),
                        B.w * (1.0f + sc.w));
      if (MOD == MOD_SHIFT_SCALE) {
        const float4 sh = ((const float4*)(mrow + shift_off))[i];
        B = make_float4(B.x + sh.x, B.y + sh.y, B.z + sh.z, B.w + sh.w);
      }
    }
  };
  bool shared = true;
  int mr0 = 0;
  if (per_row) {
    mr0 = rows[row0];
    bool same = true;
    if (t < kNormRows && row0 + t < n) same = rows[row0 + t] == mr0;
    shared = __syncthreads_and(same);
  }
  if (shared) {
    for (int i = t; i < nc; i += 64 * kNormRows) {
      float4 G, B;
      gb(mr0, i, G, B);
      gb_lds[i] = G;
      gb_lds[nc + i] = B;
    }
    __syncthreads();
  }
  if (row >= n) return;
  const float* xr = x + (size_t)row * D;
  float4 v[NCH];
  // loads clamp their chunk index (always in bounds); sums and stores skip the
  // chunks beyond the row
#pragma unroll
  for (int c = 0; c < NCH; ++c) v[c] = ld4_stream(xr + 4 * min(lane + 64 * c, nc - 1));
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < NCH; ++c)
    if (lane + 64 * c < nc)
      s += (NORM == NORM_RMS) ? (v[c].x * v[c].x + v[c].y * v[c].y + v[c].z * v[c].z + v[c].w * v[c].w)
                              : (v[c].x + v[c].y + v[c].z + v[c].w);
  s = wave_sum(s);
  float mean = 0.0f, inv;
  if (NORM == NORM_RMS) {
    inv = 1.0f / sqrtf(s / (float)D + eps);
  } else {
    mean = s / (float)D;
    float q = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      if (lane + 64 * c < nc) {
        float a = v[c].x - mean, b = v[c].y - mean, cc = v[c].z - mean, d = v[c].w - mean;
        q += a * a + b * b + cc * cc + d * d;
      }
    q = wave_sum(q);
    inv = 1.0f / sqrtf(q / (float)D + eps);
  }
  const int mr = per_row ? rows[row] : 0;
  OutT* yr = y + (size_t)row * D;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int i = lane + 64 * c;
    if (i < nc) {
      float4 G, B;
      if (shared) {
        G = gb_lds[i];
        B = gb_lds[nc + i];
      } else {
        gb(mr, i, G, B);
      }
      float4 o;
      o.x = (v[c].x - mean) * inv * G.x + B.x;
      o.y = (v[c].y - mean) * inv * G.y + B.y;
      o.z = (v[c].z - mean) * inv * G.z + B.z;
      o.w = (v[c].w - mean) * inv * G.w + B.w;
      Elt<OutT>::st4_stream(yr + 4 * i, o);
    }
  }
}

template <int NORM, int MOD, int NCH>
static void launch_norm_mod(bool out_bf16, const float* x, int n, int D, const float* g,
                            const float* beta, float eps, const float* mods, int mstride,
                            const int* rows, int so, int sc, void* y, hipStream_t s) {
  const dim3 grid((n + kNormRows - 1) / kNormRows);
  const size_t lds = (size_t)2 * (D / 4) * sizeof(float4);  // G and B: 8 D bytes
  if (out_bf16)
    k_norm_mod<NORM, MOD, NCH, bf16_t><<<grid, 64 * kNormRows, lds, s>>>(
        x, n, D, g, beta, eps, mods, mstride, rows, so, sc, (bf16_t*)y);
  else
    k_norm_mod<NORM, MOD, NCH, float><<<grid, 64 * kNormRows, lds, s>>>(
        x, n, D, g, beta, eps, mods, mstride, rows, so, sc, (float*)y);
}

template <int NORM, int MOD>
static void launch_norm_mod(bool out_bf16, const float* x, int n, int D, const float* g,
                            const float* beta, float eps, const float* mods, int mstride,
                            const int* rows, int so, int sc, void* y, hipStream_t s) {
  const int per_lane = (D + 255) / 256;  // float4 chunks per lane
#define NMC(C_) launch_norm_mod<NORM, MOD, C_>(out_bf16, x, n, D, g, beta, eps, mods, mstride, rows, so, sc, y, s)
  if (per_lane <= 4) NMC(4);
  else if (per_lane <= 8) NMC(8);
  else if (per_lane <= 12) NMC(12);
  else NMC(16);
#undef NMC
}

hipError_t norm_mod(int norm, int mod, bool out_bf16, const float* x, int n, int D, const float* g,
                    const float* beta, float eps, const float* mods, int mstride, const int* rows,
                    int shift_off, int scale_off, void* y, hipStream_t s) {
  if (n <= 0) return hipSuccess;
#define NM(N_, M_) launch_norm_mod<N_, M_>(out_bf16, x, n, D, g, beta, eps, mods, mstride, rows, shift_off, scale_off, y, s)
  if (norm == NORM_RMS) {
    if (mod == MOD_NONE) NM(NORM_RMS, MOD_NONE);
    else if (mod == MOD_SHIFT_SCALE) NM(NORM_RMS, MOD_SHIFT_SCALE);
    else NM(NORM_RMS, MOD_SCALE);
  } else {
    if (mod == MOD_NONE) NM(NORM_LAYER, MOD_NONE);
    else if (mod == MOD_SHIFT_SCALE) NM(NORM_LAYER, MOD_SHIFT_SCALE);
    else NM(NORM_LAYER, MOD_SCALE);
  }
#undef NM
  return hipGetLastError();
}

// ------------------------------------------------------------------------------
// Sandwich residual ([ZIMG] TransformerBlock.Forward):
//   x1 = x + tanh(gate) * RMSNorm(y; g_post), and when g_next is given
//   xf = RMSNorm(x1; g_next) * (1 + scale) for the next half.
// Without modulation (the context refiner) gate and scale are NULL: a plain
// residual and an unscaled pre-norm.
// ------------------------------------------------------------------------------
template <typename OutT>
__global__ __launch_bounds__(256) void k_sandwich(const float* __restrict__ x,
                                                  const float* __restrict__ y, int n, int D,
                                                  const float* __restrict__ g_post,
                                                  const float* __restrict__ gate, float eps,
                                                  float* __restrict__ x1,
                                                  const float* __restrict__ g_next,
                                                  const float* __restrict__ scale,
                                                  OutT* __restrict__ xf) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n) return;
  const int nc = D >> 2;
  const float4* yr = (const float4*)(y + (size_t)row * D);
  const float4* xr = (const float4*)(x + (size_t)row * D);
  float4 v[kMaxChunks];
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    int i = lane + 64 * c;
    if (i < nc) {
      v[c] = yr[i];
      s += v[c].x * v[c].x + v[c].y * v[c].y + v[c].z * v[c].z + v[c].w * v[c].w;
    }
  }
  float inv = 1.0f / sqrtf(wave_sum(s) / (float)D + eps);
  float s2 = 0.0f;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    int i = lane + 64 * c;
    if (i < nc) {
      float4 xx = xr[i], gp = ((const float4*)g_post)[i];
      float4 tg = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
      if (gate) {
        const float4 gt = ((const float4*)gate)[i];
        tg = make_float4(tanh_f(gt.x), tanh_f(gt.y), tanh_f(gt.z), tanh_f(gt.w));
      }
      float4 o;
      o.x = xx.x + tg.x * (v[c].x * inv * gp.x);
      o.y = xx.y + tg.y * (v[c].y * inv * gp.y);
      o.z = xx.z + tg.z * (v[c].z * inv * gp.z);
      o.w = xx.w + tg.w * (v[c].w * inv * gp.w);
      ((float4*)(x1 + (size_t)row * D))[i] = o;
      v[c] = o;
      s2 += o.x * o.x + o.y * o.y + o.z * o.z + o.w * o.w;
    }
  }
  if (g_next == nullptr) return;
  float inv2 = 1.0f / sqrtf(wave_sum(s2) / (float)D + eps);
  OutT* fr = xf + (size_t)row * D;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    int i = lane + 64 * c;
    if (i < nc) {
      float4 gn = ((const float4*)g_next)[i];
      const float4 sc = scale ? ((const float4*)scale)[i] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      float4 o;
      o.x = v[c].x * inv2 * gn.x * (1.0f + sc.x);
      o.y = v[c].y * inv2 * gn.y * (1.0f + sc.y);
      o.z = v[c].z * inv2 * gn.z * (1.0f + sc.z);
      o.w = v[c].w * inv2 * gn.w * (1.0f + sc.w);
      Elt<OutT>::st4(fr + 4 * i, o);
    }
  }
}

hipError_t sandwich(const float* x, const float* y, int n, int D, const float* g_post,
                    const float* gate, float eps, float* x1, const float* g_next,
                    const float* scale, bool xf_bf16, void* xf, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  dim3 grid((n + 3) / 4);
  if (xf_bf16)
    k_sandwich<bf16_t><<<grid, 256, 0, s>>>(x, y, n, D, g_post, gate, eps, x1, g_next, scale,
                                             (bf16_t*)xf);
  else
    k_sandwich<float><<<grid, 256, 0, s>>>(x, y, n, D, g_post, gate, eps, x1, g_next, scale,
                                            (float*)xf);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------
// RoPE table: angle (i, j) = pos[i, a] * theta^(-2m/d_a) for pair j = (axis a,
// frequency m), axes concatenated t, h, w ([MMH3] rope_angles; per-axis
// frequencies as [ZIMG] prepareRoPE3D).  A thread owns one pair j (its
// frequency is computed once, in fp64) and walks the tokens.  The angle is
// formed and reduced to [-pi, pi] in fp64, and its cosine and sine are taken in
// fp32 from there: the table is stored in fp32, and the reduced angle's fp32
// rounding (at most 2^-24 pi) keeps them within two fp32 ulps of the fp64 values.
// ------------------------------------------------------------------------------
constexpr int kRopeTokRows = 4;     // token rows of a block (blockDim = 64 x 4)
constexpr int kRopeMaxBlocks = 512;

DIT_DEV float2 cos_sin_reduced(double ang) {
  constexpr double kTwoPi = 6.283185307179586476925287;
  const double r = ang - rint(ang * (1.0 / kTwoPi)) * kTwoPi;
  float sn, cn;
  sincosf((float)r, &sn, &cn);
  return make_float2(cn, sn);
}

__global__ __launch_bounds__(64 * kRopeTokRows) void k_rope_table(
    const float* __restrict__ pos, int n, int P, int d0, int d1, int d2, double theta,
    float2* __restrict__ cs) {
  const int j = threadIdx.x & 63;
  if (j >= P) return;
  int a, m, d;
  if (j < d0 / 2) {
    a = 0; m = j; d = d0;
  } else if (j < d0 / 2 + d1 / 2) {
    a = 1; m = j - d0 / 2; d = d1;
  } else {
    a = 2; m = j - d0 / 2 - d1 / 2; d = d2;
  }
  const double omega = pow(theta, -2.0 * (double)m / (double)d);
  for (int i = blockIdx.x * kRopeTokRows + (threadIdx.x >> 6); i < n; i += gridDim.x * kRopeTokRows)
    cs[(size_t)i * P + j] = cos_sin_reduced((double)pos[(size_t)i * 3 + a] * omega);
}

static int rope_grid(int n) {
  return min((n + kRopeTokRows - 1) / kRopeTokRows, kRopeMaxBlocks);
}

hipError_t rope_table(const float* pos, int n, int P, const int axes[3], double theta, float* cs,
                      hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (P > 64) return hipErrorInvalidValue;  // one lane per rotation pair
  k_rope_table<<<rope_grid(n), 64 * kRopeTokRows, 0, s>>>(pos, n, P, axes[0], axes[1], axes[2],
                                                          theta, (float2*)cs);
  return hipGetLastError();
}

// Partial RoPE table ([MMH3] rope_angles with the checkpoint's frequency
// vector): pair j < 3k turns by pos[i, j / k] * freq[j % k]; pairs [3k, P) by
// zero (cos 1, sin 0), the head dims that stay unrotated.  fp64 angles, reduced
// as above.
__global__ __launch_bounds__(64 * kRopeTokRows) void k_rope_table_shared(
    const float* __restrict__ pos, int n, int P, int k, const float* __restrict__ freq,
    float2* __restrict__ cs) {
  const int j = threadIdx.x & 63;
  if (j >= P) return;
  const int a = j < 3 * k ? j / k : 0;
  const double f = j < 3 * k ? (double)freq[j - a * k] : 0.0;
  for (int i = blockIdx.x * kRopeTokRows + (threadIdx.x >> 6); i < n; i += gridDim.x * kRopeTokRows)
    cs[(size_t)i * P + j] = j < 3 * k ? cos_sin_reduced((double)pos[(size_t)i * 3 + a] * f)
                                      : make_float2(1.0f, 0.0f);
}

hipError_t rope_table_shared(const float* pos, int n, int P, int k, const float* freq, float* cs,
                             hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (P > 64) return hipErrorInvalidValue;
  k_rope_table_shared<<<rope_grid(n), 64 * kRopeTokRows, 0, s>>>(pos, n, P, k, freq,
                                                                 (float2*)cs);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------
// Head split of the fused qkv panel with qk-RMSNorm and RoPE on q and k
// ([MMH3] norm_rope_w; qk-norm before rotary as [ENC] rms_norm_heads).
// One wave per (token, head, q|k); lane p owns rotation pair p.  q is scaled by
// q_scale (the softmax's base-2 score scale) after the rotation.  Tokens in [n, ldn) are
// written as zeros so attention reads finite padding.
// ------------------------------------------------------------------------------
template <typename T, int HD>
__global__ __launch_bounds__(256) void k_qk_split(const T* __restrict__ qkv, int n, int ldn, int H,
                                                  const float* __restrict__ qn,
                                                  const float* __restrict__ kn, float eps,
                                                  const float2* __restrict__ cs, int rope_mode,
                                                  float q_scale, T* __restrict__ q_out,
                                                  T* __restrict__ k_out) {
  constexpr int P = HD / 2;
  const int lane = threadIdx.x & 63;
  const int tok = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int h = blockIdx.y, which = blockIdx.z;
  if (tok >= ldn) return;
  const int D = H * HD;
  T* dst = (which ? k_out : q_out) + ((size_t)h * ldn + tok) * HD;
  const bool act = lane < P;
  int ia, ib;
  if (rope_mode == 2) {
    ia = 2 * lane; ib = 2 * lane + 1;
  } else {
    ia = lane; ib = lane + P;
  }
  if (tok >= n) {
    if (act) {
      Elt<T>::st(dst + ia, 0.0f);
      Elt<T>::st(dst + ib, 0.0f);
    }
    return;
  }
  const T* src = qkv + (size_t)tok * 3 * D + which * D + h * HD;
  float a = 0.0f, b = 0.0f;
  if (act) {
    a = Elt<T>::ld(src + ia);
    b = Elt<T>::ld(src + ib);
  }
  const float* g = which ? kn : qn;
  if (g) {
    float ss = wave_sum(a * a + b * b);
    float inv = 1.0f / sqrtf(ss / (float)HD + eps);
    if (act) {
      a = a * inv * g[ia];
      b = b * inv * g[ib];
    }
  }
  if (act && rope_mode != 0) {
    float2 c = cs[(size_t)tok * P + lane];
    float ra = a * c.x - b * c.y;
    float rb = a * c.y + b * c.x;
    a = ra;
    b = rb;
  }
  if (which == 0) {
    a *= q_scale;
    b *= q_scale;
  }
  if (act) {
    Elt<T>::st(dst + ia, a);
    Elt<T>::st(dst + ib, b);
  }
}

// V part of the panel, transposed per head: vt[h, d, tok], zeros for tok >= n.
template <typename T>
__global__ __launch_bounds__(256) void k_v_transpose(const T* __restrict__ qkv, int n, int ldn,
                                                     int H, int HD, T* __restrict__ vt) {
  __shared__ float tile[64][65];
  const int t0 = blockIdx.x * 64, d0 = blockIdx.y * 64, h = blockIdx.z;
  const int D = H * HD;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int r = ty; r < 64; r += 4) {
    int tok = t0 + r;
    float v = 0.0f;
    if (tok < n) v = Elt<T>::ld(qkv + (size_t)tok * 3 * D + 2 * D + h * HD + d0 + tx);
    tile[r][tx] = v;
  }
  __syncthreads();
  for (int r = ty; r < 64; r += 4) {
    int d = d0 + r;
    int tok = t0 + tx;
    if (tok < ldn) Elt<T>::st(vt + ((size_t)h * HD + d) * ldn + tok, tile[tx][r]);
  }
}

template <typename T>
static void launch_split(int hd, const void* qkv, int n, int ldn, int H, const float* qn,
                         const float* kn, float eps, const float* cs, int rope_mode,
                         float q_scale, void* q, void* k, void* vt, hipStream_t s) {
  dim3 g1((ldn + 3) / 4, H, 2);
  if (hd == 128)
    k_qk_split<T, 128><<<g1, 256, 0, s>>>((const T*)qkv, n, ldn, H, qn, kn, eps,
                                          (const float2*)cs, rope_mode, q_scale, (T*)q, (T*)k);
  else
    k_qk_split<T, 64><<<g1, 256, 0, s>>>((const T*)qkv, n, ldn, H, qn, kn, eps,
                                         (const float2*)cs, rope_mode, q_scale, (T*)q, (T*)k);
  dim3 g2(ldn / 64, hd / 64, H);
  k_v_transpose<T><<<g2, 256, 0, s>>>((const T*)qkv, n, ldn, H, hd, (T*)vt);
}

hipError_t qk_split(int dtype, int hd, const void* qkv, int n, int ldn, int H, const float* qn,
                    const float* kn, float eps, const float* cs, int rope_mode, float q_scale,
                    void* q, void* k, void* vt, hipStream_t s) {
  if (ldn <= 0) return hipSuccess;
  if (dtype == BF16)
    launch_split<bf16_t>(hd, qkv, n, ldn, H, qn, kn, eps, cs, rope_mode, q_scale, q, k, vt, s);
  else
    launch_split<float>(hd, qkv, n, ldn, H, qn, kn, eps, cs, rope_mode, q_scale, q, k, vt, s);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------
// Weight preparation: row maps (RowMap) and scaling.
// SwiGLU group interleave of fc1 (N = 2F rows): group g = r / 64, j = r % 64;
// j < 32 -> gate row 32 g + j, else up row F + 32 g + (j - 32).
// Partial RoPE ([MMH3] norm_rope_w: pairs (j, j + P) for j < P = 3k, dims
// [2P, hd) unrotated): stored head dim d takes the page's dim d (d < P),
// d + P (P <= d < hd/2), d - (hd/2 - P) (hd/2 <= d < hd/2 + P) or d, so that
// the rotated pairs land on (j, j + hd/2) and the unrotated dims on pairs that
// the table turns by zero.
// ------------------------------------------------------------------------------
DIT_DEV int map_row(const RowMap& m, int r) {
  if (m.swiglu_F > 0) {
    int g = r >> 6, j = r & 63;
    r = (j < 32) ? (32 * g + j) : (m.swiglu_F + 32 * g + (j - 32));
  }
  if (r < m.perm_rows) {
    const int h = m.perm_hd / 2, P = m.perm_P;
    const int d = r % m.perm_hd;
    const int sd = d < P ? d : (d < h ? d + P : (d < h + P ? d - (h - P) : d));
    r += sd - d;
  }
  if (m.src_mod > 0) r %= m.src_mod;
  return r;
}

template <typename T>
__global__ void k_prep_matrix(const T* __restrict__ src, T* __restrict__ dst, int rows, int cols,
                              RowMap m, int scale_rows, float scale) {
  size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  size_t total = (size_t)rows * cols;
  if (idx >= total) return;
  int r = (int)(idx / cols), c = (int)(idx - (size_t)r * cols);
  float v = Elt<T>::ld(src + (size_t)map_row(m, r) * cols + c);
  if (r < scale_rows) v *= scale;
  Elt<T>::st(dst + idx, v);
}

hipError_t prep_matrix(int dtype, const void* src, void* dst, int rows, int cols, const RowMap& m,
                       int scale_rows, float scale, hipStream_t s) {
  size_t total = (size_t)rows * cols;
  if (total == 0) return hipSuccess;
  dim3 grid((unsigned)((total + 255) / 256));
  if (dtype == BF16)
    k_prep_matrix<bf16_t><<<grid, 256, 0, s>>>((const bf16_t*)src, (bf16_t*)dst, rows, cols, m,
                                                scale_rows, scale);
  else
    k_prep_matrix<float><<<grid, 256, 0, s>>>((const float*)src, (float*)dst, rows, cols, m,
                                               scale_rows, scale);
  return hipGetLastError();
}

hipError_t prep_matrix(int dtype, const void* src, void* dst, int rows, int cols, int swiglu_F,
                       int scale_rows, float scale, hipStream_t s) {
  RowMap m;
  m.swiglu_F = swiglu_F;
  return prep_matrix(dtype, src, dst, rows, cols, m, scale_rows, scale, s);
}

__global__ void k_prep_vector(const float* __restrict__ src, float* __restrict__ dst, int n,
                              RowMap m, int scale_n, float scale) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float v = src ? src[map_row(m, i)] : 0.0f;
  dst[i] = (i < scale_n) ? v * scale : v;
}

hipError_t prep_vector(const float* src, float* dst, int n, const RowMap& m, int scale_n,
                       float scale, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  k_prep_vector<<<(n + 255) / 256, 256, 0, s>>>(src, dst, n, m, scale_n, scale);
  return hipGetLastError();
}

hipError_t prep_vector(const float* src, float* dst, int n, int scale_n, float scale,
                       hipStream_t s) {
  return prep_vector(src, dst, n, RowMap(), scale_n, scale, s);
}

}  // namespace dit
