// Full bidirectional attention over the packed sequence, per head, without
// ever forming the score plane ([MMH3] attention: every token attends to every
// token; softmax normalisation deferred to the output as in [SIGLIP]'s
// deferred normalisation).
//
// bf16 path (flash-style, MFMA): a workgroup owns 256 queries of one head, eight
// waves of 32.  Each wave keeps its queries' Q fragment in registers and walks
// the keys in tiles of 64 staged through LDS (double-buffered):
//   S^T = K Q^T     (v_mfma_f32_32x32x16_bf16, A = K rows, B = Q^T)
//   online softmax in base 2 (max, rescale, exp2), P in bf16
//   O^T += V^T P^T  (A = V^T rows from the transposed V panel, B = P^T)
// Because S^T's accumulator layout gives every lane one query column, the
// softmax statistics are per lane and P lands in registers exactly in the
// B-operand layout of the second product once the rows of the K tile are loaded
// in a fixed permuted order (bits 2 and 3 of the row index swapped).
// When q already carries the whole base-2 score scale (UNIT), the running
// maximum is subtracted by the first MFMA of each score block (its
// accumulator input is a register block holding -m), so the exponent needs no
// per-score VALU instruction besides v_exp itself.
//
// fp32 path: a plain per-query loop (one thread per query), for the fp32
// configuration.
#include <math.h>

#include "dev_common.h"
#include "dit_kernels.h"

namespace dit {

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
constexpr bf16x2_t kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};
// Word 3 of a buffer resource for raw (unstrided, untyped) loads on gfx9-class
// parts: a 32-bit data format, so that the loads are range-checked in bytes.
constexpr int kBufferFlags = 0x00020000;

// Row permutation of a 32-key block: swap bits 2 and 3.
DIT_DEV int key_perm(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

constexpr int kAttnWaves = 8;  // 8 waves x 32 queries per workgroup
// key ranges a unit of the grid's last round splits into, at most (a shard of
// 3200 queries leaves 17 units past one round: 15 ranges fill the CUs)
constexpr int kAttnMaxSplit = 16;
constexpr int kAttnThreads = 64 * kAttnWaves;
constexpr int kAttnRows = 32 * kAttnWaves;
static_assert(kAttnRows == kAttnQueryRows, "partial-buffer rows");

// Unit u -> head h, its sample's key range [ks, ke), first query q0 and query
// end qe (the sample's end, or the query range's with one sample).  The scan
// over the table is unrolled (constant indices: scalar kernel-argument loads)
// and keeps the last sample whose first block is <= the unit's block.
DIT_DEV void unit_of(const SeqTable& t, int u, int& h, int& ks, int& ke, int& q0, int& qe) {
  const int per_head = t.blk[t.nseq];
  h = u / per_head;
  const int b = u - h * per_head;
  int b0 = 0;
  ks = t.start[0];
  ke = t.start[1];
#pragma unroll
  for (int i = 1; i < kMaxSeqs; ++i) {
    if (i < t.nseq && b >= t.blk[i]) {
      b0 = t.blk[i];
      ks = t.start[i];
      ke = t.start[i + 1];
    }
  }
  const int qs = t.nseq == 1 ? t.qlo : ks;
  qe = t.nseq == 1 ? t.qhi : ke;
  q0 = qs + (b - b0) * kAttnRows;
}

// Work units are (head, block of 256 queries of one sample), head-major, the
// query blocks of each sample starting at its first token.  A unit's queries
// attend to the keys of their sample ([ENC] attention_ragged: a ragged batch
// behaves as the sequences run alone); with one sample that is every key.
// Units below `whole` take all of their keys and write O.  The remaining units
// (the last, partial round of the grid) are each split into `nsplit`
// consecutive key ranges, one workgroup per range, which write unnormalized
// partial results (O, running maximum, row sum) for k_attn_merge to combine.
template <int HD, bool UNIT>
__global__ __launch_bounds__(kAttnThreads, 1) void k_attn_bf16(const bf16_t* __restrict__ Q,
                                                      const bf16_t* __restrict__ Kp,
                                                      const bf16_t* __restrict__ Vt, int n,
                                                      int ldn, int ldq, int H, float scale_log2,
                                                      bf16_t* __restrict__ O, int whole,
                                                      int nsplit, float* __restrict__ part,
                                                      SeqTable seqs) {
  constexpr int KT = 64;        // keys per tile
  constexpr int NC = HD / 16;   // MFMA k-steps over the head dim
  constexpr int ND = HD / 32;   // 32-row blocks of O^T
  constexpr int KCH = HD / 8;   // 16-byte chunks per K row
  constexpr int KPT = KT * KCH / kAttnThreads;  // K chunks per thread per tile
  constexpr int VPT = HD * (KT / 8) / kAttnThreads;
  // LDS rows are padded by one 16-byte chunk: the 16 rows one quarter-wave
  // reads at the same chunk then start in 16 different bank groups, and each
  // lane's addresses for the different chunks differ by constants (immediate
  // offsets of ds_read_b128 rather than one address register per chunk).
  constexpr int KLD = HD + 8, VLD = KT + 8;
  __shared__ __attribute__((aligned(16))) bf16_t sK[2][KT * KLD];
  __shared__ __attribute__((aligned(16))) bf16_t sV[2][HD * VLD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  // Workgroup i runs on XCD i % 8 and each XCD has its own L2: the whole units
  // are dealt out so that every XCD gets a contiguous run of them, whose
  // neighbours (query blocks of one head) then share that head's K/V stream in
  // the XCD's L2 (2.5x fewer bytes fetched past L2 at t2va than round-robin).
  const int whole8 = whole / 8 * 8;
  const int w = (int)blockIdx.x < whole8 ? (int)(blockIdx.x % 8) * (whole8 / 8) + (int)blockIdx.x / 8
                                         : (int)blockIdx.x;
  const bool split = w >= whole;
  const int u = split ? whole + (w - whole) / nsplit : w;
  const int j = split ? (w - whole) % nsplit : 0;
  const int ns = split ? nsplit : 1;
  int h, ks, ke, q0, qe;
  unit_of(seqs, u, h, ks, ke, q0, qe);
  q0 += wave * 32;
  // key tiles [t_lo, t_hi) of this workgroup, out of the sample's [T0, T1)
  const int T0 = ks / KT, T1 = (ke + KT - 1) / KT;
  const int t_lo = T0 + j * (T1 - T0) / ns, t_hi = T0 + (j + 1) * (T1 - T0) / ns;
  const bf16_t* Qh = Q + (size_t)h * ldq * HD;
  const bf16_t* Kh = Kp + (size_t)h * ldn * HD;
  const bf16_t* Vh = Vt + (size_t)h * HD * ldn;

  bf16x8_t qf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c)
    qf[c] = *(const bf16x8_t*)(Qh + (size_t)min(q0 - seqs.qbase + l32, ldq - 1) * HD + 16 * c + 8 * half);

  // K and V tiles arrive through buffer loads: a thread's byte offsets inside a
  // tile are fixed and the tile's position is the scalar offset, so stepping
  // to the next tile costs no vector address arithmetic.
  const __amdgpu_buffer_rsrc_t rsK =
      __builtin_amdgcn_make_buffer_rsrc((void*)Kh, (short)0, ldn * HD * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rsV =
      __builtin_amdgcn_make_buffer_rsrc((void*)Vh, (short)0, ldn * HD * 2, kBufferFlags);
  int koff[KPT], voff[VPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int c_ = tid + kAttnThreads * i;
    koff[i] = ((c_ / KCH) * HD + (c_ % KCH) * 8) * 2;
  }
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int c_ = tid + kAttnThreads * i;
    voff[i] = ((c_ / (KT / 8)) * ldn + (c_ % (KT / 8)) * 8) * 2;
  }
  u32x4_t rk[KPT], rv[VPT];
#define KOFF(row, ch) ((row) * KLD + ((ch) << 3))
#define VOFF(row, ch) ((row) * VLD + ((ch) << 3))
#define ATT_GLOAD(k0)                                                              \
  do {                                                                             \
    _Pragma("unroll") for (int i = 0; i < KPT; ++i)                                \
      rk[i] = __builtin_amdgcn_raw_buffer_load_b128(rsK, koff[i], (k0) * HD * 2, 0); \
    _Pragma("unroll") for (int i = 0; i < VPT; ++i)                                \
      rv[i] = __builtin_amdgcn_raw_buffer_load_b128(rsV, voff[i], (k0) * 2, 0);    \
  } while (0)
#define ATT_SSTORE(b)                                                              \
  do {                                                                             \
    _Pragma("unroll") for (int i = 0; i < KPT; ++i) {                              \
      int c_ = tid + kAttnThreads * i, row_ = c_ / KCH, ch_ = c_ % KCH;                     \
      *(u32x4_t*)(&sK[b][KOFF(row_, ch_)]) = rk[i];                                \
    }                                                                              \
    _Pragma("unroll") for (int i = 0; i < VPT; ++i) {                              \
      int c_ = tid + kAttnThreads * i, row_ = c_ / (KT / 8), ch_ = c_ % (KT / 8);           \
      *(u32x4_t*)(&sV[b][VOFF(row_, ch_)]) = rv[i];                                \
    }                                                                              \
  } while (0)

  f32x16_t oacc[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[d][v] = 0.0f;
  // Base-2 running maximum actually used for the exponentials.  It is only
  // raised when a tile's maximum exceeds it by more than kLazy (O and the row
  // sum are then rescaled); otherwise p = 2^(s*c - m) <= 2^kLazy, harmless in
  // the fp32 sums and in bf16, and the final normalization is unchanged.
  constexpr float kLazy = 8.0f;
  float m_run = -INFINITY;
  // row sum in four partial sums (four short dependency chains instead of one)
  float l4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  // Scores are kept relative to cm (base 2): t = s * scale_log2 - cm.  cm is
  // 0 until the first tile has set m_run, then equal to m_run.  With UNIT the
  // subtraction happens in the MFMA through cneg = {-cm, ...}.
  float cm = 0.0f;
  f32x16_t cneg;
#pragma unroll
  for (int v = 0; v < 16; ++v) cneg[v] = 0.0f;

  const int t_full = min(t_hi, ke / KT);  // tiles in [ceil(ks/KT), t_full) are all valid
  ATT_GLOAD(t_lo * KT);
  ATT_SSTORE(t_lo & 1);
  ATT_GLOAD(min(t_lo + 1, t_hi - 1) * KT);
  __syncthreads();
  const int krow = key_perm(l32);

#define ATT_TILE(MASKED)                                                                   \
  do {                                                                                     \
    f32x16_t s_[2];                                                                        \
    _Pragma("unroll") for (int kb = 0; kb < 2; ++kb) {                                     \
      _Pragma("unroll") for (int c = 0; c < NC; ++c) {                                     \
        bf16x8_t a_ = *(const bf16x8_t*)(&sK[b][KOFF(kb * 32 + krow, 2 * c + half)]);    \
        s_[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_, qf[c], c == 0 ? cneg : s_[kb], \
                                                         0, 0, 0);                         \
      }                                                                                    \
      if (!UNIT) {                                                                         \
        _Pragma("unroll") for (int v = 0; v < 16; ++v)                                     \
          s_[kb][v] = fmaf(s_[kb][v], scale_log2, -cm);                                    \
      }                                                                                    \
    }                                                                                      \
    /* value v of block kb is key kb*32 + 16*(v/8) + 8*half + v%8 of the tile */           \
    if (MASKED) {                                                                          \
      _Pragma("unroll") for (int kb = 0; kb < 2; ++kb)                                     \
      _Pragma("unroll") for (int v = 0; v < 16; ++v) {                                     \
        const int key = t * KT + kb * 32 + 16 * (v >> 3) + 8 * half + (v & 7);            \
        if (key < ks || key >= ke) s_[kb][v] = -INFINITY;                                  \
      }                                                                                    \
    }                                                                                      \
    float mx_ = -INFINITY;                                                                 \
    _Pragma("unroll") for (int kb = 0; kb < 2; ++kb)                                       \
    _Pragma("unroll") for (int v = 0; v < 16; ++v) mx_ = fmaxf(mx_, s_[kb][v]);           \
    mx_ = half_swap_max(mx_);                                                              \
    const bool need_ = cm + mx_ > m_run + kLazy;                                           \
    if (__ballot(need_)) {                                                                 \
      const float m_new_ = need_ ? cm + mx_ : m_run;                                       \
      const float alpha_ = __builtin_amdgcn_exp2f(m_run - m_new_);                         \
      const float delta_ = m_new_ - cm;                                                    \
      m_run = m_new_;                                                                      \
      cm = m_new_;                                                                         \
      _Pragma("unroll") for (int i = 0; i < 4; ++i) l4[i] *= alpha_;                      \
      _Pragma("unroll") for (int d = 0; d < ND; ++d)                                       \
      _Pragma("unroll") for (int v = 0; v < 16; ++v) oacc[d][v] *= alpha_;                 \
      _Pragma("unroll") for (int kb = 0; kb < 2; ++kb)                                     \
      _Pragma("unroll") for (int v = 0; v < 16; ++v) s_[kb][v] -= delta_;                  \
      if (UNIT) {                                                                          \
        _Pragma("unroll") for (int v = 0; v < 16; ++v) cneg[v] = -cm;                      \
      }                                                                                    \
    }                                                                                      \
    /* the row sum adds the bf16 weights the second product uses, two per  */           \
    /* v_dot2 against (1, 1); each pair is converted once, as one word      */           \
    /* (taking the words back out of the bf16x8 operand instead gave every  */           \
    /* v_dot2 of a group the same word with this compiler)                  */           \
    bf16x8_t p_[2][2];                                                                     \
    _Pragma("unroll") for (int kb = 0; kb < 2; ++kb)                                       \
    _Pragma("unroll") for (int cc = 0; cc < 2; ++cc) {                                     \
      u32x4_t w_;                                                                          \
      _Pragma("unroll") for (int q = 0; q < 4; ++q) {                                      \
        const bf16x2_t pr_ = {(__bf16)__builtin_amdgcn_exp2f(s_[kb][8 * cc + 2 * q]),      \
                              (__bf16)__builtin_amdgcn_exp2f(s_[kb][8 * cc + 2 * q + 1])}; \
        l4[q] = __builtin_amdgcn_fdot2_f32_bf16(pr_, kOnes2, l4[q], false);                \
        w_[q] = __builtin_bit_cast(unsigned, pr_);                                         \
      }                                                                                    \
      p_[kb][cc] = __builtin_bit_cast(bf16x8_t, w_);                                       \
    }                                                                                      \
    _Pragma("unroll") for (int kb = 0; kb < 2; ++kb)                                       \
    _Pragma("unroll") for (int cc = 0; cc < 2; ++cc)                                       \
    _Pragma("unroll") for (int d = 0; d < ND; ++d) {                                       \
      bf16x8_t a_ = *(const bf16x8_t*)(&sV[b][VOFF(d * 32 + l32, 4 * kb + 2 * cc + half)]); \
      oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_, p_[kb][cc], oacc[d], 0, 0, 0); \
    }                                                                                      \
  } while (0)

  // A first tile that starts before the sample (masked), the full tiles in the
  // loop, a ragged last tile (masked) after it.
  int t = t_lo;
  if (t * KT < ks) {
    const int b = t & 1;
    ATT_TILE(true);
    ATT_SSTORE(b ^ 1);
    ATT_GLOAD(min(t + 2, t_hi - 1) * KT);
    __syncthreads();
    ++t;
  }
  for (; t < t_full; ++t) {
    const int b = t & 1;
    ATT_TILE(false);
    // Unconditional (see the GEMM): tile t+1 to LDS, then the loads of t+2.
    ATT_SSTORE(b ^ 1);
    ATT_GLOAD(min(t + 2, t_hi - 1) * KT);
    __syncthreads();
  }
  if (t < t_hi) {
    const int b = t & 1;
    ATT_TILE(true);
  }
#undef ATT_TILE
#undef ATT_GLOAD
#undef ATT_SSTORE
#undef KOFF
#undef VOFF

  const float lt = half_swap_sum((l4[0] + l4[1]) + (l4[2] + l4[3]));
  const int qi = q0 + l32;
  if (split) {
    // partial slot (unit, range): O^T unnormalized fp32 [256][HD], then (m, l)
    const size_t slot = (size_t)(u - whole) * nsplit + j;
    const int ql = wave * 32 + l32;
    float* po = part + (slot * kAttnRows + ql) * HD;
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(float4*)(po + d * 32 + 8 * g + 4 * half) =
            make_float4(oacc[d][4 * g], oacc[d][4 * g + 1], oacc[d][4 * g + 2], oacc[d][4 * g + 3]);
    if (half == 0) {
      float* pml = part + (size_t)kAttnMaxSlots * kAttnRows * HD + (slot * kAttnRows + ql) * 2;
      *(float2*)pml = make_float2(m_run, lt);
    }
    return;
  }
  const float inv = 1.0f / lt;
  if (qi < qe) {
    bf16_t* orow = O + (size_t)(qi - seqs.qbase) * (H * HD) + h * HD;
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        int col = d * 32 + 8 * g + 4 * half;
        *(uint2*)(orow + col) =
            make_uint2(pack2bf(oacc[d][4 * g + 0] * inv, oacc[d][4 * g + 1] * inv),
                       pack2bf(oacc[d][4 * g + 2] * inv, oacc[d][4 * g + 3] * inv));
      }
  }
}

// Token i -> the token range [a, e) of its sample (unrolled scan, as unit_of).
DIT_DEV void sample_of(const SeqTable& t, int i, int& a, int& e) {
  a = t.start[0];
  e = t.start[1];
#pragma unroll
  for (int s = 1; s < kMaxSeqs; ++s)
    if (s < t.nseq && i >= t.start[s]) {
      a = t.start[s];
      e = t.start[s + 1];
    }
}

// fp32: one thread per query, keys in LDS tiles of 32, online softmax in base
// 2.  The block walks the keys of every sample its queries belong to; each
// thread uses only its own sample's keys.
template <int HD>
__global__ __launch_bounds__(128) void k_attn_f32(const float* __restrict__ Q,
                                                  const float* __restrict__ Kp,
                                                  const float* __restrict__ Vt, int n, int ldn,
                                                  int ldq, float scale_log2, SeqTable seqs,
                                                  float* __restrict__ O) {
  __shared__ float sk[32][HD + 1];
  __shared__ float sv[32][HD + 1];
  const int h = blockIdx.y, H = gridDim.y;
  const int b0 = seqs.qlo + blockIdx.x * 128;  // first query token of the block
  const int qi = b0 + threadIdx.x;
  int qs, qe, blo, bhi, t0, t1;
  sample_of(seqs, min(qi, n - 1), qs, qe);
  sample_of(seqs, b0, blo, t0);
  sample_of(seqs, min(b0 + 127, n - 1), t1, bhi);
  // rows past the query range read rows of q the caller padded (ldq % 128 == 0)
  const float* qr = Q + ((size_t)h * ldq + (qi - seqs.qbase)) * HD;
  float q[HD], acc[HD];
#pragma unroll
  for (int d = 0; d < HD; ++d) {
    q[d] = qr[d];
    acc[d] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;
  for (int k0 = blo & ~31; k0 < bhi; k0 += 32) {
    for (int e = threadIdx.x; e < 32 * HD; e += 128) {
      int j = e / HD, d = e % HD;
      sk[j][d] = Kp[((size_t)h * ldn + k0 + j) * HD + d];
      int d2 = e / 32, j2 = e % 32;
      sv[j2][d2] = Vt[((size_t)h * HD + d2) * ldn + k0 + j2];
    }
    __syncthreads();
    const int j0 = max(qs - k0, 0), j1 = min(qe - k0, 32);  // this query's keys in the tile
    if (j1 > j0) {
      float sc[32];
      float mx = m;
      for (int j = j0; j < j1; ++j) {
        float s = 0.0f;
#pragma unroll
        for (int d = 0; d < HD; ++d) s = fmaf(q[d], sk[j][d], s);
        sc[j] = s * scale_log2;
        mx = fmaxf(mx, sc[j]);
      }
      const float alpha = exp2f(m - mx);  // m = -inf before the first key: alpha = 0
      l *= alpha;
#pragma unroll
      for (int d = 0; d < HD; ++d) acc[d] *= alpha;
      for (int j = j0; j < j1; ++j) {
        float p = exp2f(sc[j] - mx);
        l += p;
#pragma unroll
        for (int d = 0; d < HD; ++d) acc[d] = fmaf(p, sv[j][d], acc[d]);
      }
      m = mx;
    }
    __syncthreads();
  }
  if (qi < seqs.qhi) {
    float inv = 1.0f / l;
    float* orow = O + (size_t)(qi - seqs.qbase) * (H * HD) + h * HD;
#pragma unroll
    for (int d = 0; d < HD; ++d) orow[d] = acc[d] * inv;
  }
}

// Combines the key-range partials of the split units: per query,
// M = max m_j, O = sum_j 2^(m_j - M) O_j / sum_j 2^(m_j - M) l_j.  One wave per
// query row, lanes over the head dimension.
template <int HD>
__global__ __launch_bounds__(256) void k_attn_merge(const float* __restrict__ part, int H,
                                                    int whole, int nsplit, int nunits,
                                                    SeqTable seqs, bf16_t* __restrict__ O) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);  // (split unit, query) row
  if (r >= nunits * kAttnRows) return;
  const int us = r / kAttnRows, ql = r % kAttnRows;
  int h, ks, ke, q0, qe;
  unit_of(seqs, whole + us, h, ks, ke, q0, qe);
  const int qi = q0 + ql;
  if (qi >= qe) return;
  const float* pml = part + (size_t)kAttnMaxSlots * kAttnRows * HD;
  float M = -INFINITY;
  for (int j = 0; j < nsplit; ++j)
    M = fmaxf(M, pml[(((size_t)us * nsplit + j) * kAttnRows + ql) * 2]);
  constexpr int PER = HD / 64;
  float acc[PER] = {};
  float L = 0.0f;
  for (int j = 0; j < nsplit; ++j) {
    const size_t slot = (size_t)us * nsplit + j;
    const float2 ml = *(const float2*)(pml + (slot * kAttnRows + ql) * 2);
    const float wgt = __builtin_amdgcn_exp2f(ml.x - M);
    L += wgt * ml.y;
    const float* po = part + (slot * kAttnRows + ql) * HD;
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] += wgt * po[lane * PER + e];
  }
  const float inv = 1.0f / L;
  bf16_t* orow = O + (size_t)(qi - seqs.qbase) * (H * HD) + h * HD + lane * PER;
#pragma unroll
  for (int e = 0; e < PER; ++e) orow[e] = f2bf(acc[e] * inv);
}

int device_cus() {
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cus[dev]) {
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
      c = 256;
    cus[dev] = c;
  }
  return cus[dev];
}

void make_seq_table(const int* seq_starts, int nseq, int n, SeqTable* t) {
  t->qbase = 0;
  if (!seq_starts) {
    make_shard_table(n, 0, n, t);
    return;
  }
  t->nseq = nseq;
  t->blk[0] = 0;
  for (int i = 0; i <= nseq; ++i) t->start[i] = seq_starts[i];
  for (int i = 0; i < nseq; ++i)
    t->blk[i + 1] = t->blk[i] + (seq_starts[i + 1] - seq_starts[i] + kAttnRows - 1) / kAttnRows;
  t->qlo = seq_starts[0];
  t->qhi = seq_starts[nseq];
}

void make_shard_table(int n, int qlo, int qhi, SeqTable* t) {
  t->nseq = 1;
  t->start[0] = 0;
  t->start[1] = n;
  t->blk[0] = 0;
  t->blk[1] = (qhi - qlo + kAttnRows - 1) / kAttnRows;
  t->qlo = qlo;
  t->qhi = qhi;
  t->qbase = qlo;
}

hipError_t attention(int dtype, int hd, const void* q, int ldq, const void* k, const void* vt,
                     int n, int ldn, int H, float scale_log2, void* o, float* part,
                     const SeqTable& seqs, hipStream_t s) {
  if (n <= 0 || seqs.qhi <= seqs.qlo) return hipSuccess;
  if (dtype == BF16) {
    const bf16_t *Qb = (const bf16_t*)q, *Kb = (const bf16_t*)k, *Vb = (const bf16_t*)vt;
    bf16_t* Ob = (bf16_t*)o;
    // One workgroup per CU at a time: units = H * query blocks run in rounds
    // of `cus`.  A last round that would leave at least half the CUs idle is
    // split along the keys so that it fills them (each range keeps at least
    // one key tile of the shortest sample).
    const int units = H * seqs.blk[seqs.nseq];
    if (units == 0) return hipSuccess;
    int min_tiles = 1 << 30;
    for (int i = 0; i < seqs.nseq; ++i) {
      const int a = seqs.start[i], e = seqs.start[i + 1];
      if (e > a) min_tiles = min(min_tiles, (e + 63) / 64 - a / 64);
    }
    const int cus = min(device_cus(), kAttnMaxSlots);
    const int tail = units % cus;
    int nsplit = tail ? min(min(cus / tail, kAttnMaxSplit), min_tiles) : 1;
    if (!part || nsplit < 2) nsplit = 1;
    const int whole = nsplit > 1 ? units - tail : units;
    const int grid = whole + (units - whole) * nsplit;
    const bool unit = scale_log2 == 1.0f;
#define ATT_LAUNCH(HD_, U_)                                                                      \
  k_attn_bf16<HD_, U_><<<grid, kAttnThreads, 0, s>>>(Qb, Kb, Vb, n, ldn, ldq, H, scale_log2, Ob, \
                                                     whole, nsplit, part, seqs)
    if (hd == 128 && unit) ATT_LAUNCH(128, true);
    else if (hd == 128) ATT_LAUNCH(128, false);
    else if (unit) ATT_LAUNCH(64, true);
    else ATT_LAUNCH(64, false);
#undef ATT_LAUNCH
    if (nsplit > 1) {
      const int rows = (units - whole) * kAttnRows;
      if (hd == 128)
        k_attn_merge<128><<<(rows + 3) / 4, 256, 0, s>>>(part, H, whole, nsplit, units - whole, seqs, Ob);
      else
        k_attn_merge<64><<<(rows + 3) / 4, 256, 0, s>>>(part, H, whole, nsplit, units - whole, seqs, Ob);
    }
  } else {
    dim3 grid((seqs.qhi - seqs.qlo + 127) / 128, H);
    if (hd == 128)
      k_attn_f32<128><<<grid, 128, 0, s>>>((const float*)q, (const float*)k, (const float*)vt, n,
                                           ldn, ldq, scale_log2, seqs, (float*)o);
    else
      k_attn_f32<64><<<grid, 128, 0, s>>>((const float*)q, (const float*)k, (const float*)vt, n,
                                          ldn, ldq, scale_log2, seqs, (float*)o);
  }
  return hipGetLastError();
}

}  // namespace dit
