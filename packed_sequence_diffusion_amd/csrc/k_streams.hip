// Video and audio latents <-> token rows of the packed sequence ([MMH3]
// patchify_video / unpatchify_video, pack_audio / unpack_audio):
//   video [C, T, H, W] -> rows [T*(H/2)*(W/2), 4C]: row (t, h2, w2), column
//     c*4 + p*2 + q holds x[c, t, 2*h2 + p, 2*w2 + q] (the 2 x 2 spatial patch,
//     channel-major outer);
//   audio [C, 2, T] -> rows [2T, C]: row ch*T + t, column c holds x[c, ch, t]
//     (channel 0's frames, then channel 1's);
//   with CL (channel-last columns, [ZIMG] PatchifyLatents, T = 1): column
//     (p*2 + q)*C + c holds x[c, 2*h2 + p, 2*w2 + q].
// One thread per row element on the row side, so that the rows (the GEMM
// operand, written in the GEMM dtype) are written contiguously.
#include "dev_common.h"
#include "dit_kernels.h"

namespace dit {

template <typename OutT, bool CL>
__global__ void k_patchify(const float* __restrict__ x, int C, int T, int H, int W,
                           OutT* __restrict__ rows) {
  const size_t total = (size_t)T * (H / 2) * (W / 2) * C * 4;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int col = (int)(i % (4 * C));
  const size_t r = i / (4 * C);
  const int w2 = (int)(r % (W / 2)), h2 = (int)((r / (W / 2)) % (H / 2)), t = (int)(r / ((size_t)(W / 2) * (H / 2)));
  const int c = CL ? col % C : col >> 2;
  const int pq = CL ? col / C : col & 3;
  const int p = pq >> 1, q = pq & 1;
  Elt<OutT>::st(rows + i, x[(((size_t)c * T + t) * H + 2 * h2 + p) * W + 2 * w2 + q]);
}

template <bool CL>
__global__ void k_unpatchify(const float* __restrict__ rows, int C, int T, int H, int W,
                             float* __restrict__ x) {
  const size_t total = (size_t)T * (H / 2) * (W / 2) * C * 4;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int col = (int)(i % (4 * C));
  const size_t r = i / (4 * C);
  const int w2 = (int)(r % (W / 2)), h2 = (int)((r / (W / 2)) % (H / 2)), t = (int)(r / ((size_t)(W / 2) * (H / 2)));
  const int c = CL ? col % C : col >> 2;
  const int pq = CL ? col / C : col & 3;
  const int p = pq >> 1, q = pq & 1;
  x[(((size_t)c * T + t) * H + 2 * h2 + p) * W + 2 * w2 + q] = rows[i];
}

template <typename OutT>
__global__ void k_pack_audio(const float* __restrict__ x, int C, int T, OutT* __restrict__ rows) {
  const size_t total = (size_t)2 * T * C;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int c = (int)(i % C);
  const size_t r = i / C;  // ch * T + t
  const int ch = (int)(r / T), t = (int)(r % T);
  Elt<OutT>::st(rows + i, x[((size_t)c * 2 + ch) * T + t]);
}

__global__ void k_unpack_audio(const float* __restrict__ rows, int C, int T, float* __restrict__ x) {
  const size_t total = (size_t)2 * T * C;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int c = (int)(i % C);
  const size_t r = i / C;
  const int ch = (int)(r / T), t = (int)(r % T);
  x[((size_t)c * 2 + ch) * T + t] = rows[i];
}

template <typename T>
__global__ void k_fill(T* __restrict__ p, int n, T v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

static unsigned blocks_for(size_t total) { return (unsigned)((total + 255) / 256); }

hipError_t fill_i32(int* p, int n, int v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  k_fill<int><<<blocks_for((size_t)n), 256, 0, s>>>(p, n, v);
  return hipGetLastError();
}

// rows[i] = base + tag[i], the tag clamped to the three modalities
__global__ void k_rows_from_tags(const int* __restrict__ tags, int n, int base, int* __restrict__ rows) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) rows[i] = base + min(max(tags[i], 0), 2);
}

hipError_t rows_from_tags(const int* tags, int n, int base, int* rows, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  k_rows_from_tags<<<blocks_for((size_t)n), 256, 0, s>>>(tags, n, base, rows);
  return hipGetLastError();
}

hipError_t fill_f32(float* p, int n, float v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  k_fill<float><<<blocks_for((size_t)n), 256, 0, s>>>(p, n, v);
  return hipGetLastError();
}

template <bool CL>
static hipError_t patchify_impl(int dtype, const float* x, int C, int T, int H, int W, void* rows,
                                hipStream_t s) {
  const size_t total = (size_t)T * (H / 2) * (W / 2) * C * 4;
  if (total == 0) return hipSuccess;
  if (dtype == BF16)
    k_patchify<bf16_t, CL><<<blocks_for(total), 256, 0, s>>>(x, C, T, H, W, (bf16_t*)rows);
  else
    k_patchify<float, CL><<<blocks_for(total), 256, 0, s>>>(x, C, T, H, W, (float*)rows);
  return hipGetLastError();
}

template <bool CL>
static hipError_t unpatchify_impl(const float* rows, int C, int T, int H, int W, float* x,
                                  hipStream_t s) {
  const size_t total = (size_t)T * (H / 2) * (W / 2) * C * 4;
  if (total == 0) return hipSuccess;
  k_unpatchify<CL><<<blocks_for(total), 256, 0, s>>>(rows, C, T, H, W, x);
  return hipGetLastError();
}

hipError_t patchify_video(int dtype, const float* x, int C, int T, int H, int W, void* rows,
                          hipStream_t s) {
  return patchify_impl<false>(dtype, x, C, T, H, W, rows, s);
}

hipError_t unpatchify_video(const float* rows, int C, int T, int H, int W, float* x, hipStream_t s) {
  return unpatchify_impl<false>(rows, C, T, H, W, x, s);
}

hipError_t patchify_image(int dtype, const float* x, int C, int H, int W, void* rows, hipStream_t s) {
  return patchify_impl<true>(dtype, x, C, 1, H, W, rows, s);
}

hipError_t unpatchify_image(const float* rows, int C, int H, int W, float* x, hipStream_t s) {
  return unpatchify_impl<true>(rows, C, 1, H, W, x, s);
}

hipError_t pack_audio(int dtype, const float* x, int C, int T, void* rows, hipStream_t s) {
  const size_t total = (size_t)2 * T * C;
  if (total == 0) return hipSuccess;
  if (dtype == BF16)
    k_pack_audio<bf16_t><<<blocks_for(total), 256, 0, s>>>(x, C, T, (bf16_t*)rows);
  else
    k_pack_audio<float><<<blocks_for(total), 256, 0, s>>>(x, C, T, (float*)rows);
  return hipGetLastError();
}

hipError_t unpack_audio(const float* rows, int C, int T, float* x, hipStream_t s) {
  const size_t total = (size_t)2 * T * C;
  if (total == 0) return hipSuccess;
  k_unpack_audio<<<blocks_for(total), 256, 0, s>>>(rows, C, T, x);
  return hipGetLastError();
}

}  // namespace dit
