// Successive SVID extraction of boolean kernels from a real weight ("Highly
// Efficient and Effective LLMs with Multi-Boolean Architectures", technical
// summary, section 2): item 1 approximates a matrix by its signs with a
// rank-one scale, W ~ sign(W) . (s_out s_in^T); item 3 extracts each later
// kernel the same way from the residual the earlier ones leave.
//
// Per kernel k, on the fp32 residual r (r = W for the first):
//   Wb_k      = sign(r), bit = (r >= 0), packed by the pack kernel;
//   (s, u, v) = the leading singular triplet of |r|, by power iteration
//               from the all-ones direction (|r| is nonnegative, so the
//               iterates and the limit are nonnegative: the Perron pair);
//   s_out_k   = fp16(sqrt(s) u),  s_in_k = fp16(sqrt(s) v);
//   r        -= sign(r) . (s_out_k s_in_k^T), with the rounded scales, so
//               later kernels absorb the rounding.
// The page leaves the rank-one fit open; the leading singular pair of |r|
// is the least-squares one (the residual is sign(r) . (|r| - s_out s_in^T),
// whose norm is that of |r| - s_out s_in^T).
//
// Every sum runs in a fixed order (per-thread strided sums, a fixed
// shuffle tree, chunk partials added in chunk order), so the result is
// bitwise reproducible.  Extraction is offline model conversion: the
// kernels are plain bandwidth-bound passes over the residual.
#include "dbf_internal.h"

namespace dbf {
namespace {

constexpr int kRowChunk = 256;  // rows per column-partial chunk

struct SvidWs {
  float* r;       // [N][M] residual
  float* u;       // [N]
  float* v;       // [M]
  float* part;    // [ceil(N / kRowChunk)][M] column partials
  float* rowsq;   // [N] row sums of r^2
  float* scal;    // [0] sigma of the last iteration
};

__device__ __forceinline__ float block_sum_256(float v, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// r = W as fp32; one workgroup per row.
__global__ void __launch_bounds__(256) svid_init_kernel(const void* w, int dt, int64_t M,
                                                         int64_t ldw, float* r) {
  const int64_t n = blockIdx.x;
  for (int64_t m = threadIdx.x; m < M; m += 256) r[n * M + m] = load_act(w, dt, n * ldw + m);
}

// v = 1 (the start direction of each kernel's iteration).
__global__ void __launch_bounds__(256) svid_ones_kernel(float* v, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) v[i] = 1.f;
}

// u[n] = sum_m |r[n, m]| v[m]; one workgroup per row.
__global__ void __launch_bounds__(256) svid_rows_kernel(const float* r, const float* v, int64_t M,
                                                         float* u) {
  __shared__ float red[4];
  const int64_t n = blockIdx.x;
  const float* row = r + n * M;
  float s = 0.f;
  for (int64_t m = threadIdx.x; m < M; m += 256) s += fabsf(row[m]) * v[m];
  s = block_sum_256(s, red);
  if (threadIdx.x == 0) u[n] = s;
}

// part[c][m] = sum over rows n of chunk c of |r[n, m]| u[n] (rows in order);
// grid (ceil(M / 256), chunks).
__global__ void __launch_bounds__(256) svid_cols_kernel(const float* r, const float* u, int64_t N,
                                                         int64_t M, float* part) {
  const int64_t m = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (m >= M) return;
  const int64_t n0 = static_cast<int64_t>(blockIdx.y) * kRowChunk;
  const int64_t n1 = min(N, n0 + kRowChunk);
  float s = 0.f;
  for (int64_t n = n0; n < n1; ++n) s += fabsf(r[n * M + m]) * u[n];
  part[static_cast<int64_t>(blockIdx.y) * M + m] = s;
}

// v[m] = sum_c part[c][m], chunks in order.
__global__ void __launch_bounds__(256) svid_colsum_kernel(const float* part, int64_t M, int nch,
                                                           float* v) {
  const int64_t m = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (m >= M) return;
  float s = 0.f;
  for (int c = 0; c < nch; ++c) s += part[static_cast<int64_t>(c) * M + m];
  v[m] = s;
}

// x /= ||x|| (left as is when ||x|| = 0); the norm goes to *norm_out if
// given.  One workgroup.
__global__ void __launch_bounds__(256) svid_normalize_kernel(float* x, int64_t n, float* norm_out) {
  __shared__ float red[4];
  float s = 0.f;
  for (int64_t i = threadIdx.x; i < n; i += 256) s += x[i] * x[i];
  s = block_sum_256(s, red);
  const float nrm = sqrtf(s);
  if (nrm > 0.f) {
    const float inv = 1.f / nrm;
    for (int64_t i = threadIdx.x; i < n; i += 256) x[i] *= inv;
  }
  if (norm_out && threadIdx.x == 0) *norm_out = nrm;
}

// s_out = fp16(sqrt(sigma) u), s_in = fp16(sqrt(sigma) v).
__global__ void __launch_bounds__(256) svid_scales_kernel(const float* u, const float* v,
                                                           const float* sigma, int64_t N, int64_t M,
                                                           uint16_t* s_out, uint16_t* s_in) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const float rs = sqrtf(*sigma);
  if (i < N) s_out[i] = f32_to_f16_bits(rs * u[i]);
  if (i < M) s_in[i] = f32_to_f16_bits(rs * v[i]);
}

// r[n, m] -= sign(r[n, m]) s_out[n] s_in[m] with the stored fp16 scales (the
// product of two fp16 values is exact in fp32); rowsq[n] = sum_m r[n, m]^2
// after the update.  One workgroup per row.
__global__ void __launch_bounds__(256) svid_update_kernel(float* r, int64_t M, const uint16_t* s_out,
                                                           const uint16_t* s_in, float* rowsq) {
  __shared__ float red[4];
  const int64_t n = blockIdx.x;
  float* row = r + n * M;
  const float so = f16_bits_to_f32(s_out[n]);
  float q = 0.f;
  for (int64_t m = threadIdx.x; m < M; m += 256) {
    const float x = row[m];
    const float p = so * f16_bits_to_f32(s_in[m]);
    const float y = x >= 0.f ? x - p : x + p;
    row[m] = y;
    q += y * y;
  }
  q = block_sum_256(q, red);
  if (threadIdx.x == 0) rowsq[n] = q;
}

// out = sum_n rowsq[n], rows in order of a fixed tree.  One workgroup.
__global__ void __launch_bounds__(256) svid_total_kernel(const float* rowsq, int64_t N, float* out) {
  __shared__ float red[4];
  float s = 0.f;
  for (int64_t i = threadIdx.x; i < N; i += 256) s += rowsq[i];
  s = block_sum_256(s, red);
  if (threadIdx.x == 0) *out = s;
}

SvidWs svid_layout(void* ws, int64_t N, int64_t M) {
  auto al = [](size_t n) { return (n + 255) / 256 * 256; };
  unsigned char* b = static_cast<unsigned char*>(ws);
  SvidWs w;
  size_t off = 0;
  w.r = reinterpret_cast<float*>(b + off); off += al(static_cast<size_t>(N) * M * 4);
  w.u = reinterpret_cast<float*>(b + off); off += al(static_cast<size_t>(N) * 4);
  w.v = reinterpret_cast<float*>(b + off); off += al(static_cast<size_t>(M) * 4);
  const int64_t nch = (N + kRowChunk - 1) / kRowChunk;
  w.part = reinterpret_cast<float*>(b + off); off += al(static_cast<size_t>(nch) * M * 4);
  w.rowsq = reinterpret_cast<float*>(b + off); off += al(static_cast<size_t>(N) * 4);
  w.scal = reinterpret_cast<float*>(b + off);
  return w;
}

}  // namespace

size_t svid_ws_bytes(int64_t N, int64_t M) {
  auto al = [](size_t n) { return (n + 255) / 256 * 256; };
  const int64_t nch = (N + kRowChunk - 1) / kRowChunk;
  return al(static_cast<size_t>(N) * M * 4) + al(static_cast<size_t>(N) * 4) +
         al(static_cast<size_t>(M) * 4) + al(static_cast<size_t>(nch) * M * 4) +
         al(static_cast<size_t>(N) * 4) + 256;
}

hipError_t launch_svid(const void* w, int w_dtype, int64_t N, int64_t M, int64_t ldw, int n_kernels,
                       uint32_t* const* wb, uint16_t* const* s_in, uint16_t* const* s_out, int iters,
                       float* residual_sq, void* ws, hipStream_t s) {
  const SvidWs b = svid_layout(ws, N, M);
  const unsigned gn = static_cast<unsigned>(N);
  const unsigned gm = static_cast<unsigned>((M + 255) / 256);
  const unsigned gnm = static_cast<unsigned>((std::max(N, M) + 255) / 256);
  const int nch = static_cast<int>((N + kRowChunk - 1) / kRowChunk);
  svid_init_kernel<<<gn, 256, 0, s>>>(w, w_dtype, M, ldw, b.r);
  hipError_t e = hipGetLastError();
  for (int k = 0; k < n_kernels && e == hipSuccess; ++k) {
    e = launch_pack(b.r, DBF_F32, N, M, M, wb[k], s);
    if (e != hipSuccess) break;
    // each kernel's iteration starts from the all-ones direction
    svid_ones_kernel<<<gm, 256, 0, s>>>(b.v, M);
    svid_normalize_kernel<<<1, 256, 0, s>>>(b.v, M, nullptr);
    for (int it = 0; it < iters; ++it) {
      svid_rows_kernel<<<gn, 256, 0, s>>>(b.r, b.v, M, b.u);
      svid_normalize_kernel<<<1, 256, 0, s>>>(b.u, N, nullptr);
      svid_cols_kernel<<<dim3(gm, static_cast<unsigned>(nch)), 256, 0, s>>>(b.r, b.u, N, M, b.part);
      svid_colsum_kernel<<<gm, 256, 0, s>>>(b.part, M, nch, b.v);
      svid_normalize_kernel<<<1, 256, 0, s>>>(b.v, M, b.scal);
    }
    svid_scales_kernel<<<gnm, 256, 0, s>>>(b.u, b.v, b.scal, N, M, s_out[k], s_in[k]);
    if (k + 1 < n_kernels || residual_sq) {
      svid_update_kernel<<<gn, 256, 0, s>>>(b.r, M, s_out[k], s_in[k], b.rowsq);
      if (residual_sq) svid_total_kernel<<<1, 256, 0, s>>>(b.rowsq, N, residual_sq + k);
    }
    e = hipGetLastError();
  }
  return e;
}

}  // namespace dbf
