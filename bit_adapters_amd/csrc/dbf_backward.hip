// Backward of the double-binary layer: dx and the gradients of the three
// scale vectors of every term, by the chain rule through the LoRDBA
// parametrization (section 2, "Arquitetura Central").  Per term i and token:
//
//   forward  u = gamma . x, s = B2 u, w = beta . s, z = B1 w, y += alpha . z
//   backward g = B1^T (alpha . dy), h = B2^T (beta . g)
//   dalpha_i = sum_t dy . z,  dbeta_i = sum_t s . g,  dgamma_i = sum_t x . h,
//   dx = sum_i gamma_i . h_i
//
// s, z, g and h are each one sign-accumulate product scale_out . (S
// (scale_in . v)) -- the boolean-kernel product with a unit output scale --
// over B2, B1, B1^T and B2^T (the transposes packed by
// dbf_transpose_packed), so they run on the decode or MFMA product kernels.
// The token sums then run here, in fixed order: column partials over chunks
// of kTokChunk tokens, then the chunks in order.
#include <algorithm>

#include "dbf_internal.h"

namespace dbf {
namespace {

constexpr int64_t kTokChunk = 64;
constexpr int kTokRound = 8;

__global__ void __launch_bounds__(256) fill_ones_f16(uint16_t* p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) p[i] = 0x3C00u;  // 1.0
}

// Column partials of the three scale gradients.  Column space: [L][N] for
// alpha, then [L][R] for beta, then [L][M] for gamma; chunk = blockIdx.y.
struct PartArgs {
  int L;
  int64_t T, N, M, R;
  const void* x;
  int x_dtype;
  int64_t ldx;
  const void* dy;
  int dy_dtype;
  int64_t lddy;
  const float *s, *z, *g, *h;  // [L][T][R], [L][T][N], [L][T][R], [L][T][M]
  float* part;                 // [chunks][L (N + R + M)]
};

// Four activations at element i (i a multiple of 4): one 16-byte load for
// fp32, one 8-byte load for bf16 / f16.
__device__ __forceinline__ float4 load4_act(const void* p, int dt, int64_t i) {
  if (dt == DBF_F32) return *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
  const uint2 v = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
  const uint16_t h[4] = {uint16_t(v.x), uint16_t(v.x >> 16), uint16_t(v.y), uint16_t(v.y >> 16)};
  float f[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) f[e] = dt == DBF_BF16 ? bf16_bits_to_f32(h[e]) : f16_bits_to_f32(h[e]);
  return make_float4(f[0], f[1], f[2], f[3]);
}

// Four adjacent columns of one segment and term per thread (every segment
// length a multiple of 4, dy and x rows aligned for load4_act); the same
// sums as grad_partial_kernel.
__global__ void __launch_bounds__(256) grad_partial4_kernel(PartArgs p) {
  const int64_t ncol = p.L * (p.N + p.R + p.M);
  const int64_t col = 4 * (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x);
  if (col >= ncol) return;
  const int64_t t0 = static_cast<int64_t>(blockIdx.y) * kTokChunk;
  const int64_t t1 = min(p.T, t0 + kTokChunk);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  auto fma4 = [&](const float4 a, const float4 b) {
    acc.x += a.x * b.x; acc.y += a.y * b.y; acc.z += a.z * b.z; acc.w += a.w * b.w;
  };
  // kTokRound tokens a round: their loads are issued together, then added
  // in token order (one round trip per round instead of per token)
  auto run = [&](auto ld_a, auto ld_b) {
    int64_t t = t0;
    for (; t + kTokRound <= t1; t += kTokRound) {
      float4 a[kTokRound], b[kTokRound];
#pragma unroll
      for (int u = 0; u < kTokRound; ++u) {
        a[u] = ld_a(t + u);
        b[u] = ld_b(t + u);
      }
#pragma unroll
      for (int u = 0; u < kTokRound; ++u) fma4(a[u], b[u]);
    }
    for (; t < t1; ++t) fma4(ld_a(t), ld_b(t));
  };
  int64_t c = col;
  if (c < p.L * p.N) {  // dalpha: dy . z
    const int64_t i = c / p.N, n = c - i * p.N;
    const float* z = p.z + i * p.T * p.N + n;
    run([&](int64_t t) { return load4_act(p.dy, p.dy_dtype, t * p.lddy + n); },
        [&](int64_t t) { return *reinterpret_cast<const float4*>(z + t * p.N); });
  } else if ((c -= p.L * p.N) < p.L * p.R) {  // dbeta: s . g
    const int64_t i = c / p.R, r = c - i * p.R;
    const float* s = p.s + i * p.T * p.R + r;
    const float* g = p.g + i * p.T * p.R + r;
    run([&](int64_t t) { return *reinterpret_cast<const float4*>(s + t * p.R); },
        [&](int64_t t) { return *reinterpret_cast<const float4*>(g + t * p.R); });
  } else {  // dgamma: x . h
    c -= p.L * p.R;
    const int64_t i = c / p.M, m = c - i * p.M;
    const float* h = p.h + i * p.T * p.M + m;
    run([&](int64_t t) { return load4_act(p.x, p.x_dtype, t * p.ldx + m); },
        [&](int64_t t) { return *reinterpret_cast<const float4*>(h + t * p.M); });
  }
  *reinterpret_cast<float4*>(p.part + static_cast<int64_t>(blockIdx.y) * ncol + col) = acc;
}

__global__ void __launch_bounds__(256) grad_partial_kernel(PartArgs p) {
  const int64_t ncol = p.L * (p.N + p.R + p.M);
  const int64_t col = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (col >= ncol) return;
  const int64_t t0 = static_cast<int64_t>(blockIdx.y) * kTokChunk;
  const int64_t t1 = min(p.T, t0 + kTokChunk);
  float acc = 0.f;
  int64_t c = col;
  if (c < p.L * p.N) {  // dalpha: dy . z
    const int64_t i = c / p.N, n = c - i * p.N;
    const float* z = p.z + i * p.T * p.N + n;
    for (int64_t t = t0; t < t1; ++t)
      acc += load_act(p.dy, p.dy_dtype, t * p.lddy + n) * z[t * p.N];
  } else if ((c -= p.L * p.N) < p.L * p.R) {  // dbeta: s . g
    const int64_t i = c / p.R, r = c - i * p.R;
    const float* s = p.s + i * p.T * p.R + r;
    const float* g = p.g + i * p.T * p.R + r;
    for (int64_t t = t0; t < t1; ++t) acc += s[t * p.R] * g[t * p.R];
  } else {  // dgamma: x . h
    c -= p.L * p.R;
    const int64_t i = c / p.M, m = c - i * p.M;
    const float* h = p.h + i * p.T * p.M + m;
    for (int64_t t = t0; t < t1; ++t)
      acc += load_act(p.x, p.x_dtype, t * p.ldx + m) * h[t * p.M];
  }
  p.part[static_cast<int64_t>(blockIdx.y) * ncol + col] = acc;
}

// Sum of the chunk partials in chunk order into the (optional) outputs.
__global__ void __launch_bounds__(256) grad_final_kernel(const float* part, int64_t ncol,
                                                          int nchunks, int L, int64_t N,
                                                          int64_t R, int64_t M, float* dalpha,
                                                          float* dbeta, float* dgamma) {
  const int64_t col = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (col >= ncol) return;
  // eight chunks' loads in flight at a time, added in chunk order
  float acc = 0.f;
  int q = 0;
  for (; q + 8 <= nchunks; q += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = part[(q + u) * ncol + col];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += v[u];
  }
  for (; q < nchunks; ++q) acc += part[q * ncol + col];
  int64_t c = col;
  if (c < L * N) {
    if (dalpha) dalpha[c] = acc;
  } else if ((c -= L * N) < L * R) {
    if (dbeta) dbeta[c] = acc;
  } else if (dgamma) {
    dgamma[c - L * R] = acc;
  }
}

// dx[t][m .. m + 4) = sum_i gamma_i[m ..] h_i[t][m ..], in term order (M a
// multiple of 4).
__global__ void __launch_bounds__(256) grad_dx4_kernel(const float* h, int L, int64_t T,
                                                        int64_t M, TermPtrs tp, void* dx,
                                                        int dx_dtype, int64_t lddx) {
  const int64_t idx = 4 * (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x);
  if (idx >= T * M) return;
  const int64_t t = idx / M, m = idx - t * M;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < L; ++i) {
    const float4 hv = *reinterpret_cast<const float4*>(h + (i * T + t) * M + m);
    const float hs[4] = {hv.x, hv.y, hv.z, hv.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += f16_bits_to_f32(tp.gamma[i][m + e]) * hs[e];
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) store_out(dx, dx_dtype, t * lddx + m + e, acc[e], 0);
}

// dx[t][m] = sum_i gamma_i[m] h_i[t][m], in term order.
__global__ void __launch_bounds__(256) grad_dx_kernel(const float* h, int L, int64_t T,
                                                       int64_t M, TermPtrs tp, void* dx,
                                                       int dx_dtype, int64_t lddx) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= T * M) return;
  const int64_t t = idx / M, m = idx - t * M;
  float acc = 0.f;
  for (int i = 0; i < L; ++i) acc += f16_bits_to_f32(tp.gamma[i][m]) * h[(i * T + t) * M + m];
  store_out(dx, dx_dtype, t * lddx + m, acc, 0);
}

int64_t al256(int64_t n) { return (n + 255) / 256 * 256; }

// One product out [T x rows] (fp32) = S (scale_in . v): S packed with K
// columns, unit output scale.
struct Product {
  const uint32_t* bits;
  int64_t rows, K;
};

size_t product_ws(const Product& q, int64_t T, int path) {
  return path == DBF_PATH_MFMA ? mfma_bool_ws_bytes(q.rows, q.K, 1, T)
                               : decode_ws_bytes(q.rows, q.K, q.rows, 1, T);
}

hipError_t run_product(const Product& q, const uint16_t* scale_in, const uint16_t* ones,
                       const void* v, int v_dtype, int64_t ldv, int64_t T, float* out,
                       int path, void* ws, hipStream_t s) {
  TermPtrs tp{};
  tp.n = 1;
  tp.b1[0] = tp.b2[0] = q.bits;
  tp.gamma[0] = scale_in;
  tp.alpha[0] = tp.beta[0] = ones;
  if (path == DBF_PATH_MFMA)
    return launch_bool_mfma(tp, q.rows, q.K, v, v_dtype, T, ldv, out, DBF_F32, q.rows, 0, ws, s);
  return launch_bool_decode(tp, q.rows, q.K, v, v_dtype, T, ldv, out, DBF_F32, q.rows, 0, ws, s);
}

struct BwdLayout {
  size_t scratch, ones, s, z, g, h, part, total;
};

BwdLayout bwd_layout(int64_t N, int64_t M, int64_t R, int L, int64_t T, int path) {
  BwdLayout w{};
  // the products' own scratch follows the shared head; ours follows theirs
  size_t sc = kWsHeadBytes;
  const Product shapes[4] = {{nullptr, R, M}, {nullptr, N, R}, {nullptr, R, N}, {nullptr, M, R}};
  for (const Product& q : shapes) sc = std::max(sc, product_ws(q, T, path));
  size_t off = al256(static_cast<int64_t>(sc));
  w.scratch = sc;
  w.ones = off; off += al256(2 * std::max(std::max(N, M), R));
  w.s = off; off += al256(4 * L * T * R);
  w.z = off; off += al256(4 * L * T * N);
  w.g = off; off += al256(4 * L * T * R);
  w.h = off; off += al256(4 * L * T * M);
  const int64_t nchunks = (T + kTokChunk - 1) / kTokChunk;
  w.part = off; off += al256(4 * nchunks * L * (N + R + M));
  w.total = off;
  return w;
}

}  // namespace

size_t backward_ws_bytes(int64_t N, int64_t M, int64_t R, int n_terms, int64_t T, int path) {
  return bwd_layout(N, M, R, n_terms, T, path).total;
}

hipError_t launch_backward(const TermPtrs& t, const uint32_t* const* b1t,
                           const uint32_t* const* b2t, int64_t N, int64_t M, int64_t R,
                           const void* x, int x_dtype, int64_t ldx, const void* dy,
                           int dy_dtype, int64_t lddy, int64_t T, void* dx, int dx_dtype,
                           int64_t lddx, float* dalpha, float* dbeta, float* dgamma,
                           int path, void* ws, hipStream_t s) {
  unsigned char* base = static_cast<unsigned char*>(ws);
  const BwdLayout lay = bwd_layout(N, M, R, t.n, T, path);
  uint16_t* ones = reinterpret_cast<uint16_t*>(base + lay.ones);
  float* sv = reinterpret_cast<float*>(base + lay.s);
  float* zv = reinterpret_cast<float*>(base + lay.z);
  float* gv = reinterpret_cast<float*>(base + lay.g);
  float* hv = reinterpret_cast<float*>(base + lay.h);
  const int64_t nones = std::max(std::max(N, M), R);
  fill_ones_f16<<<dim3(static_cast<unsigned>((nones + 255) / 256)), 256, 0, s>>>(ones, nones);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  for (int i = 0; i < t.n; ++i) {
    float* si = sv + i * T * R;
    float* zi = zv + i * T * N;
    float* gi = gv + i * T * R;
    float* hi = hv + i * T * M;
    // s = B2 (gamma . x); z = B1 (beta . s); g = B1^T (alpha . dy); h = B2^T (beta . g)
    if ((e = run_product({t.b2[i], R, M}, t.gamma[i], ones, x, x_dtype, ldx, T, si, path, ws, s)))
      return e;
    if ((e = run_product({t.b1[i], N, R}, t.beta[i], ones, si, DBF_F32, R, T, zi, path, ws, s)))
      return e;
    if ((e = run_product({b1t[i], R, N}, t.alpha[i], ones, dy, dy_dtype, lddy, T, gi, path, ws, s)))
      return e;
    if ((e = run_product({b2t[i], M, R}, t.beta[i], ones, gi, DBF_F32, R, T, hi, path, ws, s)))
      return e;
  }
  if (dalpha || dbeta || dgamma) {
    PartArgs pa{};
    pa.L = t.n; pa.T = T; pa.N = N; pa.M = M; pa.R = R;
    pa.x = x; pa.x_dtype = x_dtype; pa.ldx = ldx;
    pa.dy = dy; pa.dy_dtype = dy_dtype; pa.lddy = lddy;
    pa.s = sv; pa.z = zv; pa.g = gv; pa.h = hv;
    pa.part = reinterpret_cast<float*>(base + lay.part);
    const int64_t ncol = t.n * (N + R + M);
    const int nchunks = static_cast<int>((T + kTokChunk - 1) / kTokChunk);
    // four columns a thread when no group of four crosses a segment or term
    // and dy rows are 16-byte aligned fp32
    auto rows4 = [](const void* p, int dt, int64_t ld) {
      return ld % 4 == 0 && reinterpret_cast<uintptr_t>(p) % (dt == DBF_F32 ? 16 : 8) == 0;
    };
    const bool four = N % 4 == 0 && R % 4 == 0 && M % 4 == 0 && rows4(dy, dy_dtype, lddy) &&
                      rows4(x, x_dtype, ldx);
    if (four)
      grad_partial4_kernel<<<dim3(static_cast<unsigned>((ncol / 4 + 255) / 256), nchunks), 256, 0, s>>>(pa);
    else
      grad_partial_kernel<<<dim3(static_cast<unsigned>((ncol + 255) / 256), nchunks), 256, 0, s>>>(pa);
    grad_final_kernel<<<dim3(static_cast<unsigned>((ncol + 255) / 256)), 256, 0, s>>>(
        pa.part, ncol, nchunks, t.n, N, R, M, dalpha, dbeta, dgamma);
    if ((e = hipGetLastError())) return e;
  }
  if (dx && M % 4 == 0) {
    grad_dx4_kernel<<<dim3(static_cast<unsigned>((T * M / 4 + 255) / 256)), 256, 0, s>>>(
        hv, t.n, T, M, t, dx, dx_dtype, lddx);
    if ((e = hipGetLastError())) return e;
  } else if (dx) {
    grad_dx_kernel<<<dim3(static_cast<unsigned>((T * M + 255) / 256)), 256, 0, s>>>(
        hv, t.n, T, M, t, dx, dx_dtype, lddx);
    if ((e = hipGetLastError())) return e;
  }
  return hipSuccess;
}

}  // namespace dbf
