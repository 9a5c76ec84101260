// Decode path of the double-binary layer: the two sign-accumulate products
// of LoRDBA section 2 ("Kernel de Inferencia") and DBF section 2
// ("Inferencia") done over the packed bits with additions only.
//
// Masked sum with 16-entry tables.  For each group of four consecutive
// activations a0..a3 and each 4-bit sign pattern n the table holds
//     E[n] = sum_j (bit j of n ? +a_j : -a_j) = 2 * sum_{bit j set} a_j - sum_j a_j,
// i.e. the identity  sum_k s_k a_k = 2 sum_{s_k=+1} a_k - sum_k a_k  applied
// per group, with the -sum folded into every entry.  A row's sign product is
// then one table lookup and one add per nibble of its packed bits.
//
// Mapping.  A workgroup is 4 wavefronts over one 64-row tile of the sign
// matrix; lane = row, so a wave reads one contiguous tile of kw*256 bytes
// per K-block and all 64 lanes look up the same group's 16 entries at the
// same time (16 distinct LDS banks, duplicates broadcast: conflict-free).
// The 4 waves take 4 consecutive K-blocks per pass; the tables of a pass are
// built cooperatively in LDS, and wave partials are reduced in LDS in a
// fixed order (no atomics, bitwise reproducible).
//
// Stage 1 (B2, rows = R, K = M): t = B2 (gamma . x), w = beta . t, written
// to the workspace as fp32 (or exact int32 S1 for int8 activations).  The K
// range may be split over several workgroups (ks partials, summed in a fixed
// order by stage 2) to put enough workgroups on the chip when R is small.
// Stage 2 (B1, rows = N, K = R): z = B1 w summed over the terms with alpha,
// y written once per token.
#include "dbf_internal.h"

namespace dbf {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxKS = 8;

enum { S1_FLOAT = 0, S1_INT = 1 };
enum { S2_FLOAT = 0, S2_I8_BETA = 1, S2_INT = 2 };

template <typename A>
__device__ __forceinline__ void build_signed16(A a0, A a1, A a2, A a3, A* e) {
  const A p0 = -a0 - a1, p1 = a0 - a1, p2 = a1 - a0, p3 = a0 + a1;
  const A q0 = -a2 - a3, q1 = a2 - a3, q2 = a3 - a2, q3 = a2 + a3;
  e[0] = p0 + q0;  e[1] = p1 + q0;  e[2] = p2 + q0;  e[3] = p3 + q0;
  e[4] = p0 + q1;  e[5] = p1 + q1;  e[6] = p2 + q1;  e[7] = p3 + q1;
  e[8] = p0 + q2;  e[9] = p1 + q2;  e[10] = p2 + q2; e[11] = p3 + q2;
  e[12] = p0 + q3; e[13] = p1 + q3; e[14] = p2 + q3; e[15] = p3 + q3;
}

template <int KW>
__device__ __forceinline__ void load_row_words(const uint32_t* p, uint32_t* wd) {
  if constexpr (KW == 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    wd[0] = v.x; wd[1] = v.y; wd[2] = v.z; wd[3] = v.w;
  } else if constexpr (KW == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    wd[0] = v.x; wd[1] = v.y;
  } else {
#pragma unroll
    for (int w = 0; w < KW; ++w) wd[w] = p[w];
  }
}

// Lookups of one lane's KW words against the tables of its wave's K-block.
template <typename A, int TB, int KW>
__device__ __forceinline__ void lookup(const A* tb, int gpp, const uint32_t* wd,
                                       A* acc) {
#pragma unroll
  for (int w = 0; w < KW; ++w) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int nib = (wd[w] >> (4 * c)) & 15;
#pragma unroll
      for (int tok = 0; tok < TB; ++tok)
        acc[tok] += tb[(tok * gpp + w * 8 + c) * 16 + nib];
    }
  }
}

struct S1Args {
  TermPtrs t;
  const void* x;
  int x_dtype;
  int64_t ldx, T, R, M, nkb, kb_per_split;
  int ks;
  void* ws;
  int64_t rs;
  int32_t* s1_out;  // int variant only (ks == 1)
};

template <typename A, int TB, int KW, int MODE>
__global__ void __launch_bounds__(kThreads)
stage1_kernel(S1Args p) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int gpp = kWaves * 8 * KW;  // 4-groups per pass
  A* tbl = reinterpret_cast<A*>(smem);  // [TB][gpp][16]
  A* red = tbl + TB * gpp * 16;         // [kWaves][TB][64]
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t rt = blockIdx.x;
  const int split = blockIdx.y, term = blockIdx.z;
  const uint32_t* bits = p.t.b2[term];
  const uint16_t* gam = p.t.gamma[term];
  const uint16_t* bet = p.t.beta[term];
  const int64_t kb_begin = static_cast<int64_t>(split) * p.kb_per_split;
  const int64_t kb_end = min(p.nkb, kb_begin + p.kb_per_split);
  const int64_t row = rt * 64 + lane;

  for (int64_t tok0 = 0; tok0 < p.T; tok0 += TB) {
    A acc[TB];
#pragma unroll
    for (int i = 0; i < TB; ++i) acc[i] = A(0);
    for (int64_t kb0 = kb_begin; kb0 < kb_end; kb0 += kWaves) {
      const int64_t kb = kb0 + wv;
      uint32_t wd[KW];
#pragma unroll
      for (int w = 0; w < KW; ++w) wd[w] = 0;
      if (kb < kb_end)
        load_row_words<KW>(bits + ((rt * p.nkb + kb) * 64 + lane) * KW, wd);
      const int64_t kbase = kb0 * 32 * KW;
      for (int e = threadIdx.x; e < TB * gpp; e += kThreads) {
        const int tok = e / gpp, g = e - tok * gpp;
        const int64_t tt = tok0 + tok;
        const int64_t k = kbase + 4 * g;
        A a[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          a[j] = A(0);
          if (tt < p.T && k + j < p.M) {
            if constexpr (MODE == S1_INT) {
              a[j] = static_cast<const int8_t*>(p.x)[tt * p.ldx + k + j];
            } else {
              a[j] = f16_bits_to_f32(gam[k + j]) *
                     load_act(p.x, p.x_dtype, tt * p.ldx + k + j);
            }
          }
        }
        build_signed16<A>(a[0], a[1], a[2], a[3], tbl + (tok * gpp + g) * 16);
      }
      __syncthreads();
      if (kb < kb_end) lookup<A, TB, KW>(tbl + wv * 8 * KW * 16, gpp, wd, acc);
      __syncthreads();
    }
#pragma unroll
    for (int tok = 0; tok < TB; ++tok) red[(wv * TB + tok) * 64 + lane] = acc[tok];
    __syncthreads();
    if (wv == 0 && row < p.R) {
#pragma unroll
      for (int tok = 0; tok < TB; ++tok) {
        const int64_t tt = tok0 + tok;
        if (tt >= p.T) break;
        A t = red[tok * 64 + lane];
#pragma unroll
        for (int v = 1; v < kWaves; ++v) t += red[(v * TB + tok) * 64 + lane];
        const int64_t o = ((static_cast<int64_t>(term) * p.ks + split) * p.T + tt) * p.rs + row;
        if constexpr (MODE == S1_INT) {
          static_cast<int32_t*>(p.ws)[o] = t;
          if (p.s1_out) p.s1_out[(term * p.T + tt) * p.R + row] = t;
        } else {
          static_cast<float*>(p.ws)[o] = f16_bits_to_f32(bet[row]) * t;
        }
      }
    }
    __syncthreads();
  }
}

struct S2Args {
  TermPtrs t;
  int64_t T, N, R, nkb;
  int ks;
  const void* ws;
  int64_t rs;
  void* y;
  int y_dtype;
  int64_t ldy;
  int accumulate;
  int32_t* s2_out;  // S2_INT only
};

template <typename A, int TB, int KW, int MODE>
__global__ void __launch_bounds__(kThreads)
stage2_kernel(S2Args p) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int gpp = kWaves * 8 * KW;
  A* tbl = reinterpret_cast<A*>(smem);
  A* red = tbl + TB * gpp * 16;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t rt = blockIdx.x;
  const int64_t row = rt * 64 + lane;

  for (int64_t tok0 = 0; tok0 < p.T; tok0 += TB) {
    float yacc[TB];
#pragma unroll
    for (int i = 0; i < TB; ++i) yacc[i] = 0.f;
    for (int term = 0; term < p.t.n; ++term) {
      const uint32_t* bits = p.t.b1[term];
      A acc[TB];
#pragma unroll
      for (int i = 0; i < TB; ++i) acc[i] = A(0);
      for (int64_t kb0 = 0; kb0 < p.nkb; kb0 += kWaves) {
        const int64_t kb = kb0 + wv;
        uint32_t wd[KW];
#pragma unroll
        for (int w = 0; w < KW; ++w) wd[w] = 0;
        if (kb < p.nkb)
          load_row_words<KW>(bits + ((rt * p.nkb + kb) * 64 + lane) * KW, wd);
        const int64_t kbase = kb0 * 32 * KW;
        for (int e = threadIdx.x; e < TB * gpp; e += kThreads) {
          const int tok = e / gpp, g = e - tok * gpp;
          const int64_t tt = tok0 + tok;
          const int64_t k = kbase + 4 * g;
          A a[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            a[j] = A(0);
            if (tt < p.T && k + j < p.R) {
              const int64_t base = (static_cast<int64_t>(term) * p.ks * p.T + tt) * p.rs + k + j;
              if constexpr (MODE == S2_FLOAT) {
                const float* wsf = static_cast<const float*>(p.ws);
                float s = wsf[base];
                for (int q = 1; q < p.ks; ++q) s += wsf[base + q * p.T * p.rs];
                a[j] = s;
              } else if constexpr (MODE == S2_I8_BETA) {
                const int32_t* wsi = static_cast<const int32_t*>(p.ws);
                a[j] = f16_bits_to_f32(p.t.beta[term][k + j]) *
                       static_cast<float>(wsi[base]);
              } else {
                a[j] = static_cast<const int32_t*>(p.ws)[base];
              }
            }
          }
          build_signed16<A>(a[0], a[1], a[2], a[3], tbl + (tok * gpp + g) * 16);
        }
        __syncthreads();
        if (kb < p.nkb) lookup<A, TB, KW>(tbl + wv * 8 * KW * 16, gpp, wd, acc);
        __syncthreads();
      }
#pragma unroll
      for (int tok = 0; tok < TB; ++tok) red[(wv * TB + tok) * 64 + lane] = acc[tok];
      __syncthreads();
      if (wv == 0 && row < p.N) {
        const uint16_t* al = p.t.alpha[term];
        const float a_n = al ? f16_bits_to_f32(al[row]) : 1.0f;
#pragma unroll
        for (int tok = 0; tok < TB; ++tok) {
          A z = red[tok * 64 + lane];
#pragma unroll
          for (int v = 1; v < kWaves; ++v) z += red[(v * TB + tok) * 64 + lane];
          if constexpr (MODE == S2_INT) {
            const int64_t tt = tok0 + tok;
            if (tt < p.T && p.s2_out) p.s2_out[(term * p.T + tt) * p.N + row] = z;
          }
          yacc[tok] += a_n * static_cast<float>(z);
        }
      }
      __syncthreads();
    }
    if (wv == 0 && row < p.N && p.y) {
#pragma unroll
      for (int tok = 0; tok < TB; ++tok) {
        const int64_t tt = tok0 + tok;
        if (tt < p.T) store_out(p.y, p.y_dtype, tt * p.ldy + row, yacc[tok], p.accumulate);
      }
    }
  }
}

template <typename A>
size_t smem_bytes(int tb, int kw) {
  return sizeof(A) * (static_cast<size_t>(tb) * kWaves * 8 * kw * 16 +
                      static_cast<size_t>(kWaves) * tb * 64);
}

int pick_tb(int64_t T) { return T <= 1 ? 1 : (T == 2 ? 2 : 4); }

// Splits of stage 1 along K so that about 512 workgroups run.
int pick_ks(int64_t nrt, int n_terms, int64_t nkb, int64_t* kb_per_split) {
  int64_t want = 512 / std::max<int64_t>(1, nrt * n_terms);
  int64_t maxks = std::max<int64_t>(1, nkb / kWaves);
  int64_t ks = std::min<int64_t>(std::min<int64_t>(want, maxks), kMaxKS);
  if (ks < 1) ks = 1;
  int64_t per = (nkb + ks - 1) / ks;
  per = (per + kWaves - 1) / kWaves * kWaves;
  ks = (nkb + per - 1) / per;
  *kb_per_split = per;
  return static_cast<int>(ks);
}

#define DBF_TB_KW_SWITCH(TB, KW, ...)                                  \
  switch ((TB) * 8 + (KW)) {                                           \
    case 1 * 8 + 1: { constexpr int TB_ = 1, KW_ = 1; __VA_ARGS__; } break; \
    case 1 * 8 + 2: { constexpr int TB_ = 1, KW_ = 2; __VA_ARGS__; } break; \
    case 1 * 8 + 3: { constexpr int TB_ = 1, KW_ = 3; __VA_ARGS__; } break; \
    case 1 * 8 + 4: { constexpr int TB_ = 1, KW_ = 4; __VA_ARGS__; } break; \
    case 2 * 8 + 1: { constexpr int TB_ = 2, KW_ = 1; __VA_ARGS__; } break; \
    case 2 * 8 + 2: { constexpr int TB_ = 2, KW_ = 2; __VA_ARGS__; } break; \
    case 2 * 8 + 3: { constexpr int TB_ = 2, KW_ = 3; __VA_ARGS__; } break; \
    case 2 * 8 + 4: { constexpr int TB_ = 2, KW_ = 4; __VA_ARGS__; } break; \
    case 4 * 8 + 1: { constexpr int TB_ = 4, KW_ = 1; __VA_ARGS__; } break; \
    case 4 * 8 + 2: { constexpr int TB_ = 4, KW_ = 2; __VA_ARGS__; } break; \
    case 4 * 8 + 3: { constexpr int TB_ = 4, KW_ = 3; __VA_ARGS__; } break; \
    default: { constexpr int TB_ = 4, KW_ = 4; __VA_ARGS__; } break;       \
  }

template <typename A, int MODE>
hipError_t run_stage1(const TermPtrs& t, int64_t M, int64_t R, const void* x,
                      int x_dtype, int64_t T, int64_t ldx, void* ws,
                      int32_t* s1_out, bool allow_split, int* ks_out,
                      hipStream_t s) {
  S1Args a{};
  a.t = t; a.x = x; a.x_dtype = x_dtype; a.ldx = ldx; a.T = T; a.R = R; a.M = M;
  a.nkb = layout_nkb(M);
  const int64_t nrt = layout_nrt(R);
  int64_t per = 0;
  a.ks = allow_split ? pick_ks(nrt, t.n, a.nkb, &per) : 1;
  if (!allow_split) per = a.nkb;
  a.kb_per_split = per;
  a.ws = ws; a.rs = ws_rstride(R); a.s1_out = s1_out;
  *ks_out = a.ks;
  const int tb = pick_tb(T), kw = static_cast<int>(layout_kw(M));
  const dim3 grid(static_cast<unsigned>(nrt), a.ks, t.n);
  DBF_TB_KW_SWITCH(tb, kw, {
    stage1_kernel<A, TB_, KW_, MODE><<<grid, kThreads, smem_bytes<A>(TB_, KW_), s>>>(a);
  });
  return hipGetLastError();
}

template <typename A, int MODE>
hipError_t run_stage2(const TermPtrs& t, int64_t N, int64_t R, int64_t T,
                      const void* ws, int ks, void* y, int y_dtype,
                      int64_t ldy, int accumulate, int32_t* s2_out,
                      hipStream_t s) {
  S2Args a{};
  a.t = t; a.T = T; a.N = N; a.R = R; a.nkb = layout_nkb(R); a.ks = ks;
  a.ws = ws; a.rs = ws_rstride(R); a.y = y; a.y_dtype = y_dtype; a.ldy = ldy;
  a.accumulate = accumulate; a.s2_out = s2_out;
  const int tb = pick_tb(T), kw = static_cast<int>(layout_kw(R));
  const dim3 grid(static_cast<unsigned>(layout_nrt(N)));
  DBF_TB_KW_SWITCH(tb, kw, {
    stage2_kernel<A, TB_, KW_, MODE><<<grid, kThreads, smem_bytes<A>(TB_, KW_), s>>>(a);
  });
  return hipGetLastError();
}

}  // namespace

size_t decode_ws_bytes(int64_t /*N*/, int64_t /*M*/, int64_t R, int n_terms,
                       int64_t T) {
  return static_cast<size_t>(n_terms) * kMaxKS * static_cast<size_t>(T) *
         static_cast<size_t>(ws_rstride(R)) * 4u;
}

hipError_t launch_decode(const TermPtrs& t, int64_t N, int64_t M, int64_t R,
                         const void* x, int x_dtype, int64_t T, int64_t ldx,
                         void* y, int y_dtype, int64_t ldy, int accumulate,
                         void* ws, hipStream_t s) {
  int ks = 1;
  hipError_t e = run_stage1<float, S1_FLOAT>(t, M, R, x, x_dtype, T, ldx, ws,
                                              nullptr, true, &ks, s);
  if (e != hipSuccess) return e;
  return run_stage2<float, S2_FLOAT>(t, N, R, T, ws, ks, y, y_dtype, ldy,
                                     accumulate, nullptr, s);
}

hipError_t launch_decode_stage1(const TermPtrs& t, int64_t M, int64_t R,
                                const void* x, int x_dtype, int64_t T,
                                int64_t ldx, void* ws, hipStream_t s) {
  int ks = 1;
  return run_stage1<float, S1_FLOAT>(t, M, R, x, x_dtype, T, ldx, ws, nullptr,
                                     true, &ks, s);
}

int decode_stage1_splits(int64_t M, int64_t R, int n_terms) {
  int64_t per = 0;
  return pick_ks(layout_nrt(R), n_terms, layout_nkb(M), &per);
}

hipError_t launch_decode_i8(const TermPtrs& t, int64_t N, int64_t M, int64_t R,
                            const int8_t* x, int64_t T, int64_t ldx,
                            int32_t* s1, int32_t* s2, void* y, int y_dtype,
                            int64_t ldy, void* ws, hipStream_t s) {
  int ks = 1;
  hipError_t e = run_stage1<int32_t, S1_INT>(t, M, R, x, DBF_I8, T, ldx, ws,
                                             s1, false, &ks, s);
  if (e != hipSuccess) return e;
  if (!s2 && !y) return hipSuccess;
  const bool beta_one = t.beta[0] == nullptr;
  if (beta_one)
    return run_stage2<int32_t, S2_INT>(t, N, R, T, ws, 1, y, y_dtype, ldy, 0,
                                       s2, s);
  return run_stage2<float, S2_I8_BETA>(t, N, R, T, ws, 1, y, y_dtype, ldy, 0,
                                       nullptr, s);
}

}  // namespace dbf
