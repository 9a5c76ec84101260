// LoRDBA adapter mode: y = W0 x + sum_i alpha_i . B1_i w_i, the adapter kept
// unmerged beside the frozen base (LoRDBA sections 1 and 5), where
// w_i = beta_i . B2_i (gamma_i . x) comes from the decode path's first stage.
//
// One workgroup owns 16 output rows.  Its 4 wavefronts split the input
// features in four and stream their quarter of the 16 bf16 W0 rows straight
// into v_mfma_f32_16x16x32_bf16 (A = W0 rows as stored, B = up to 16 tokens
// of x), so the base costs no VALU work; partials are summed in LDS in a
// fixed order.  The adapter's second sign-accumulate for the same 16 rows
// (R bits per row) and the alpha scale run in the epilogue, and y is written
// once.  Token counts above 16 are handled 16 at a time.
#include "dbf_internal.h"

namespace dbf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

struct AdArgs {
  const uint16_t* w0;
  int64_t ldw;
  TermPtrs t;
  int64_t N, M, R, T, ldx;
  const uint16_t* x;
  void* y;
  int y_dtype;
  int64_t ldy;
  const float* ws;
  int ks;
  int64_t rs;
  int64_t kq;  // features per wave (multiple of 32)
  int vec;     // 16-byte loads allowed
};

__device__ __forceinline__ uint4 load8(const uint16_t* p, int64_t k, int64_t K,
                                       bool valid, bool vec) {
  if (!valid) return make_uint4(0, 0, 0, 0);
  if (vec && k + 8 <= K) return *reinterpret_cast<const uint4*>(p + k);
  uint16_t v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = (k + j < K) ? p[k + j] : uint16_t(0);
  return make_uint4(v[0] | (uint32_t(v[1]) << 16), v[2] | (uint32_t(v[3]) << 16),
                    v[4] | (uint32_t(v[5]) << 16), v[6] | (uint32_t(v[7]) << 16));
}

__global__ void __launch_bounds__(256) adapter_kernel(AdArgs p) {
  __shared__ float red[4][16][16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int li = lane & 15, lq = lane >> 4;
  const int64_t arow = n0 + li;
  const bool arow_ok = arow < p.N;
  const uint16_t* wrow = p.w0 + (arow_ok ? arow : 0) * p.ldw;
  const int64_t kbeg = wv * p.kq;
  const int64_t kend = min(p.M, kbeg + p.kq);
  const bool vec = p.vec != 0;

  for (int64_t tb0 = 0; tb0 < p.T; tb0 += 16) {
    const int64_t tok = tb0 + li;
    const bool tok_ok = tok < p.T;
    const uint16_t* xrow = p.x + (tok_ok ? tok : 0) * p.ldx;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    int64_t k0 = kbeg;
    for (; k0 + 4 * 32 <= kend; k0 += 4 * 32) {
      uint4 a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t k = k0 + u * 32 + lq * 8;
        a[u] = load8(wrow, k, p.M, arow_ok, vec);
        b[u] = load8(xrow, k, p.M, tok_ok, vec);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, a[u]), __builtin_bit_cast(bf16x8, b[u]),
            acc, 0, 0, 0);
    }
    for (; k0 < kend; k0 += 32) {
      const int64_t k = k0 + lq * 8;
      const bool in = k < kend;
      const uint4 a = load8(wrow, k, kend, arow_ok && in, vec);
      const uint4 b = load8(xrow, k, kend, tok_ok && in, vec);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
    }
    // D[i][j]: row i = 4 * (lane / 16) + r, token j = lane % 16.
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wv][4 * lq + r][li] = acc[r];
    __syncthreads();
    {
      const int i = tid >> 4, j = tid & 15;
      const int64_t n = n0 + i, tt = tb0 + j;
      float v = red[0][i][j] + red[1][i][j] + red[2][i][j] + red[3][i][j];
      if (n < p.N && tt < p.T) {
        const int64_t rt = n >> 6, rin = n & 63;
        const int64_t kw = layout_kw(p.R), nkb = layout_nkb(p.R);
        for (int term = 0; term < p.t.n; ++term) {
          const uint32_t* b1 = p.t.b1[term];
          const float* wbase = p.ws + (static_cast<int64_t>(term) * p.ks * p.T + tt) * p.rs;
          float z = 0.f;
          for (int64_t r0 = 0; r0 < p.R; r0 += 32) {
            const int64_t kb = r0 / (32 * kw), w = (r0 % (32 * kw)) / 32;
            const uint32_t word = b1[((rt * nkb + kb) * 64 + rin) * kw + w];
            const int64_t rend = min<int64_t>(32, p.R - r0);
            for (int64_t j2 = 0; j2 < rend; ++j2) {
              float wr = wbase[r0 + j2];
              for (int q = 1; q < p.ks; ++q) wr += wbase[q * p.T * p.rs + r0 + j2];
              z += ((word >> j2) & 1u) ? wr : -wr;
            }
          }
          v += f16_bits_to_f32(p.t.alpha[term][n]) * z;
        }
        store_out(p.y, p.y_dtype, tt * p.ldy + n, v, 0);
      }
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_adapter(const uint16_t* w0, int64_t ldw, const TermPtrs& t,
                          int64_t N, int64_t M, int64_t R, const void* x,
                          int64_t T, int64_t ldx, void* y, int y_dtype,
                          int64_t ldy, const void* ws, int ks, hipStream_t s) {
  AdArgs a{};
  a.w0 = w0; a.ldw = ldw; a.t = t; a.N = N; a.M = M; a.R = R; a.T = T;
  a.ldx = ldx; a.x = static_cast<const uint16_t*>(x); a.y = y;
  a.y_dtype = y_dtype; a.ldy = ldy; a.ws = static_cast<const float*>(ws);
  a.ks = ks; a.rs = ws_rstride(R);
  a.kq = ((M + 3) / 4 + 31) / 32 * 32;
  a.vec = (ldw % 8 == 0) && (ldx % 8 == 0) &&
          (reinterpret_cast<uintptr_t>(w0) % 16 == 0) &&
          (reinterpret_cast<uintptr_t>(x) % 16 == 0);
  const dim3 grid(static_cast<unsigned>((N + 15) / 16));
  adapter_kernel<<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace dbf
