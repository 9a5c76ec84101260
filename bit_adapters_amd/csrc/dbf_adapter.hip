// LoRDBA adapter mode in one launch: y = W0 x + sum_i alpha_i . B1_i w_i,
// w_i = beta_i . B2_i (gamma_i . x), the adapter kept unmerged beside the
// frozen base (LoRDBA sections 1 and 5).
//
// Workgroups [0, n1) run the decode path's stage 1 (dbf_lut.h) for the
// adapter's B2 and publish w.  Workgroups [n1, n1 + ceil(N / 16)) own 16
// output rows each: their 8 wavefronts split the input features in eight and
// stream their share of the 16 bf16 W0 rows straight into
// v_mfma_f32_16x16x32_bf16 (A = W0 rows as stored, B = up to 16 tokens of
// x), 8 loads deep, so the base costs no VALU work and keeps HBM busy; only
// then do they wait for stage 1, which has long finished, stage w in LDS,
// and add alpha . (B1 w) for their rows before writing y once.  Token counts
// above 16 are handled 16 at a time (the base is re-streamed per 16 tokens;
// this kernel is for decode batches).
#include "dbf_lut.h"

namespace dbf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kUnroll = 8;  // W0 loads in flight per lane
constexpr int kRChunk = 256;  // ranks of w staged in LDS at a time

struct Main {
  const uint16_t* w0;
  int64_t ldw;
  TermPtrs t;
  int64_t N, M, R, T, ldx;
  const uint16_t* x;
  void* y;
  int y_dtype;
  int64_t ldy;
  const float* ws;  // stage-1 partials [L][ks][T][rs]
  int ks;
  int64_t rs;
  int64_t kq;  // features per wave (multiple of 32)
  int vec;     // 16-byte loads allowed
  unsigned* ctr;
  unsigned n1, nmain;
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

constexpr int kMainWaves = lut::kWaves;
constexpr int kMainThreads = lut::kThreads;

__device__ __forceinline__ void main_role(const Main& p, int64_t blk, float* lds) {
  // [waves][16][16] partials of the base, then w staged as [16][kRChunk]
  float (*red)[16][16] = reinterpret_cast<float (*)[16][16]>(lds);
  float* wst = lds + kMainWaves * 16 * 16;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t n0 = blk * 16;
  const int li = lane & 15, lq = lane >> 4;
  const int64_t arow = n0 + li;
  const bool arow_ok = arow < p.N;
  const uint16_t* wrow = p.w0 + (arow_ok ? arow : 0) * p.ldw;
  const int64_t kbeg = wv * p.kq;
  const int64_t kend = min(p.M, kbeg + p.kq);
  const bool vec = p.vec != 0;
  bool waited = false;

  for (int64_t tb0 = 0; tb0 < p.T; tb0 += 16) {
    const int64_t tok = tb0 + li;
    const bool tok_ok = tok < p.T;
    const uint16_t* xrow = p.x + (tok_ok ? tok : 0) * p.ldx;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    int64_t k0 = kbeg;
    for (; k0 + kUnroll * 32 <= kend; k0 += kUnroll * 32) {
      uint4 a[kUnroll], b[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t k = k0 + u * 32 + lq * 8;
        a[u] = load8(wrow, k, p.M, arow_ok, vec);
        b[u] = load8(xrow, k, p.M, tok_ok, vec);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, a[u]), __builtin_bit_cast(bf16x8, b[u]), acc, 0, 0, 0);
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
    // threads [0, 256) own one (row, token) each from here on
    const bool owner = tid < 256;
    const int i = (tid >> 4) & 15, j = tid & 15;
    const int64_t n = n0 + i, tt = tb0 + j;
    float v = 0.f;
#pragma unroll
    for (int q = 0; q < kMainWaves; ++q) v += red[q][i][j];

    if (p.t.n > 0) {
      if (!waited) {
        lut::wait_producers(p.ctr, p.n1);
        waited = true;
      }
      const int64_t kw = layout_kw(p.R), nkb = layout_nkb(p.R);
      const int64_t rt = n >> 6, rin = n & 63;
      for (int term = 0; term < p.t.n; ++term) {
        float z = 0.f;
        for (int64_t r0 = 0; r0 < p.R; r0 += kRChunk) {
          const int nr = static_cast<int>(min<int64_t>(kRChunk, p.R - r0));
          // w[tok][r0 .. r0 + nr) summed over the K-split partials
          for (int e = tid; e < 16 * nr; e += kMainThreads) {
            const int jt = e / nr, rr = e - jt * nr;
            const int64_t t2 = tb0 + jt;
            float s = 0.f;
            if (t2 < p.T) {
              const float* src = p.ws + (static_cast<int64_t>(term) * p.ks * p.T + t2) * p.rs + r0 + rr;
              float q[lut::kMaxKS];
#pragma unroll
              for (int qq = 0; qq < lut::kMaxKS; ++qq)
                if (qq < p.ks) q[qq] = src[qq * p.T * p.rs];
              s = q[0];
#pragma unroll
              for (int qq = 1; qq < lut::kMaxKS; ++qq)
                if (qq < p.ks) s += q[qq];
            }
            wst[jt * kRChunk + rr] = s;
          }
          __syncthreads();
          if (owner && n < p.N && tt < p.T) {
            const uint32_t* b1 = p.t.b1[term];
            for (int r1 = 0; r1 < nr; r1 += 32) {
              const int64_t r = r0 + r1;
              const int64_t kb = r / (32 * kw), w = (r % (32 * kw)) / 32;
              const uint32_t word = b1[((rt * nkb + kb) * 64 + rin) * kw + w];
              const int rend = min(32, nr - r1);
              const float* wr = wst + j * kRChunk + r1;
              for (int j2 = 0; j2 < rend; ++j2) z += ((word >> j2) & 1u) ? wr[j2] : -wr[j2];
            }
          }
          __syncthreads();
        }
        if (n < p.N) v += f16_bits_to_f32(p.t.alpha[term][n]) * z;
      }
    }
    if (owner && n < p.N && tt < p.T) store_out(p.y, p.y_dtype, tt * p.ldy + n, v, 0);
    __syncthreads();
  }
  if (waited) lut::consumer_done(p.ctr, p.nmain);
}

__global__ void __launch_bounds__(kMainThreads) adapter_base_only(Main m) {
  extern __shared__ __align__(16) unsigned char smem[];
  main_role(m, blockIdx.x, reinterpret_cast<float*>(smem));
}

template <int TB, int KW>
__global__ void __launch_bounds__(kMainThreads) adapter_fused(lut::Stage1 s1, Main m, int n1) {
  extern __shared__ __align__(16) unsigned char smem[];
  if (static_cast<int>(blockIdx.x) < n1) {
    float* tbl = reinterpret_cast<float*>(smem);
    float* red = tbl + lut::tbl_elems<TB, KW>();
    lut::stage1_role<float, TB, KW, lut::MODE_F>(s1, blockIdx.x, tbl, red);
    lut::publish(m.ctr);
    return;
  }
  main_role(m, static_cast<int64_t>(blockIdx.x) - n1, reinterpret_cast<float*>(smem));
}

}  // namespace

hipError_t launch_adapter(const uint16_t* w0, int64_t ldw, const TermPtrs& t,
                          int64_t N, int64_t M, int64_t R, const void* x,
                          int64_t T, int64_t ldx, void* y, int y_dtype,
                          int64_t ldy, void* ws, hipStream_t s) {
  Main m{};
  m.w0 = w0; m.ldw = ldw; m.t = t; m.N = N; m.M = M; m.R = R; m.T = T;
  m.ldx = ldx; m.x = static_cast<const uint16_t*>(x); m.y = y;
  m.y_dtype = y_dtype; m.ldy = ldy;
  m.kq = ((M + kMainWaves - 1) / kMainWaves + 31) / 32 * 32;
  m.vec = (ldw % 8 == 0) && (ldx % 8 == 0) &&
          (reinterpret_cast<uintptr_t>(w0) % 16 == 0) &&
          (reinterpret_cast<uintptr_t>(x) % 16 == 0);
  m.nmain = static_cast<unsigned>((N + 15) / 16);
  const size_t main_lds = sizeof(float) * (kMainWaves * 16 * 16 + 16 * kRChunk);
  if (t.n == 0) {
    adapter_base_only<<<dim3(m.nmain), kMainThreads, main_lds, s>>>(m);
    return hipGetLastError();
  }
  int n1 = 0;
  const lut::Stage1 a = make_stage1(t, M, R, x, DBF_BF16, T, ldx, ws, true, &n1);
  m.ws = static_cast<const float*>(a.ws);
  m.ks = a.ks;
  m.rs = a.rs;
  m.ctr = static_cast<unsigned*>(ws);
  m.n1 = static_cast<unsigned>(n1);
  const int tb = lut::pick_tb(T), kw = static_cast<int>(layout_kw(M));
  const dim3 grid(static_cast<unsigned>(n1) + m.nmain);
#define DBF_AD(TB_, KW_)                                                                 \
  adapter_fused<TB_, KW_><<<grid, kMainThreads, std::max(main_lds, lut::lds_bytes<float, TB_, KW_>()), \
                            s>>>(a, m, n1)
#define DBF_AD_KW(TB_)              \
  switch (kw) {                     \
    case 1: DBF_AD(TB_, 1); break;  \
    case 2: DBF_AD(TB_, 2); break;  \
    case 3: DBF_AD(TB_, 3); break;  \
    default: DBF_AD(TB_, 4); break; \
  }
  switch (tb) {
    case 1: DBF_AD_KW(1); break;
    case 2: DBF_AD_KW(2); break;
    default: DBF_AD_KW(4); break;
  }
#undef DBF_AD_KW
#undef DBF_AD
  return hipGetLastError();
}

}  // namespace dbf
