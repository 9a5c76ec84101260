// LoRDBA adapter mode in one launch: y = W0 x + sum_i alpha_i . B1_i w_i,
// w_i = beta_i . B2_i (gamma_i . x), the adapter kept unmerged beside the
// frozen base (LoRDBA sections 1 and 5).
//
// A row workgroup owns 16 output rows; its 8 wavefronts split the input
// features in eight and stream their share of the 16 bf16 W0 rows straight
// into v_mfma_f32_16x16x32_bf16 (A = W0 rows as stored, B = up to 16 tokens
// of x), so the base product costs no VALU work.  Token counts above 16 are
// handled 16 at a time (the base is re-streamed per 16 tokens: this kernel
// serves decode batches).
//
// Small adapters (at most 2 terms and L * ceil(R / 16) <= 4; LoRDBA uses one
// term of rank 16 to 64): each row workgroup also derives the whole
// intermediate w itself, on the matrix cores, from the x fragments it already
// holds.  The A operand is +-gamma over 16 ranks: gamma split exactly into two
// bf16 values, the signs flipped by the packed B2 bits, so every product is
// exact and the sums are fp32.  That adds at most 8 MFMAs per 32 features to
// the base's one, needs no other workgroup, no workspace and no wait, and the
// wavefronts load one group of features ahead of their MFMAs.  One token
// (decode) has a kernel of its own, adapter_tok1: stream waves copy W0 into
// LDS by DMA (or, for four rank tiles, read it into registers) while rank
// waves derive w beside them (see there).
//
// Larger adapters: workgroups [0, n1) run the decode path's stage 1
// (dbf_lut.h) for B2 and publish w; the row workgroups stream the base, then
// wait for stage 1 (long finished by then), stage w in LDS and add
// alpha . (B1 w) before writing y once.
#include "dbf_lut.h"

namespace dbf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
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
  lut::Sync sync;  // n_prod = stage-1 workgroups, n_cons = row workgroups
  unsigned nmain;
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

// 16 bytes at p + k (k + 8 within the row).  Rows past N or T are read as
// row 0 and not zeroed: an MFMA output element depends on one A row and one
// B column only, and the outputs of those rows and tokens are never stored.
// Without a branch the loads stay in flight across the MFMAs.
__device__ __forceinline__ uint4 load16(const uint16_t* p, int64_t k) {
  return *reinterpret_cast<const uint4*>(p + k);
}

// Eight waves: the row roles need more than the 128 registers per wave that
// a 1024-thread workgroup leaves.  The stage-1 roles of these kernels run
// with the same eight.
constexpr int kMainWaves = 8;
constexpr int kMainThreads = 64 * kMainWaves;

// MULTI: each token has its own adapter (tab, idx; one term each) instead of
// the terms p.t shared by every token.
// (ptrs: [kMaxAdapters] B1 then [kMaxAdapters] alpha pointers in LDS.)
template <bool MULTI = false>
__device__ __forceinline__ void main_role(const Main& p, int64_t blk, float* lds,
                                          const void* const* ptrs = nullptr, int nad = 0,
                                          const int32_t* idx = nullptr) {
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
    // two loops rather than a choice per load: the bounded loads branch per
    // lane, and a load under a branch makes the compiler wait for every
    // load before the next (kUnroll round trips per step instead of one)
    if (vec) {
      for (; k0 + kUnroll * 32 <= kend; k0 += kUnroll * 32) {
        uint4 a[kUnroll], b[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          const int64_t k = k0 + u * 32 + lq * 8;
          a[u] = load16(wrow, k);
          b[u] = load16(xrow, k);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, a[u]), __builtin_bit_cast(bf16x8, b[u]), acc, 0, 0, 0);
      }
    } else {
      for (; k0 + kUnroll * 32 <= kend; k0 += kUnroll * 32) {
        uint4 a[kUnroll], b[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          const int64_t k = k0 + u * 32 + lq * 8;
          a[u] = load8(wrow, k, p.M, arow_ok, false);
          b[u] = load8(xrow, k, p.M, tok_ok, false);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, a[u]), __builtin_bit_cast(bf16x8, b[u]), acc, 0, 0, 0);
      }
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

    if (MULTI || p.t.n > 0) {
      const int64_t kw = layout_kw(p.R), nkb = layout_nkb(p.R);
      const int64_t rt = n >> 6, rin = n & 63;
      bool active = owner && n < p.N && tt < p.T;
      // The words of this owner's B1 row for one chunk of ranks, issued
      // together (one at a time, each cost a round trip of its own).
      constexpr int kWords = kRChunk / 32;
      uint32_t wd[kWords];
      auto load_words = [&](const uint32_t* b1, int64_t r0, int nr) {
#pragma unroll
        for (int q = 0; q < kWords; ++q) {
          wd[q] = 0u;
          const int64_t r = r0 + 32 * q;
          if (active && 32 * q < nr) {
            const int64_t kb = r / (32 * kw), w = (r % (32 * kw)) / 32;
            wd[q] = b1[((rt * nkb + kb) * 64 + rin) * kw + w];
          }
        }
      };
      // one adapter for every token: the first chunk's words before the
      // wait, so their round trip overlaps it
      if constexpr (!MULTI) load_words(p.t.b1[0], 0, static_cast<int>(min<int64_t>(kRChunk, p.R)));
      if (!waited) {
        // the partials are read with system-scope loads (written through by
        // the producers), so no acquire (an L2 invalidation) is needed
        lut::wait_producers(p.sync, false);
        waited = true;
      }
      // this owner's adapter (MULTI; -1: none)
      int am = -1;
      if constexpr (MULTI) {
        if (owner && tt < p.T) {
          am = idx[tt];
          if (am < -1 || am >= nad) am = -1;  // flagged by the stage-1 workgroups
        }
        active = active && am >= 0;
      }
      const int nterms = MULTI ? 1 : p.t.n;
      for (int term = 0; term < nterms; ++term) {
        float z = 0.f;
        for (int64_t r0 = 0; r0 < p.R; r0 += kRChunk) {
          const int nr = static_cast<int>(min<int64_t>(kRChunk, p.R - r0));
          if (!MULTI && (term > 0 || r0 > 0)) load_words(p.t.b1[term], r0, nr);
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
                if (qq < p.ks)
                  q[qq] = __hip_atomic_load(src + qq * p.T * p.rs, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_SYSTEM);
              s = q[0];
#pragma unroll
              for (int qq = 1; qq < lut::kMaxKS; ++qq)
                if (qq < p.ks) s += q[qq];
            }
            wst[jt * kRChunk + rr] = s;
          }
          __syncthreads();
          // a token's own adapter: its words once its index has arrived
          if constexpr (MULTI) load_words(static_cast<const uint32_t*>(ptrs[am >= 0 ? am : 0]), r0, nr);
          if (active) {
#pragma unroll
            for (int q = 0; q < kWords; ++q) {
              if (32 * q >= nr) break;
              const uint32_t word = wd[q];
              const int rend = min(32, nr - 32 * q);
              const float* wr = wst + j * kRChunk + 32 * q;
              for (int j2 = 0; j2 < rend; ++j2) z += ((word >> j2) & 1u) ? wr[j2] : -wr[j2];
            }
          }
          __syncthreads();
        }
        if constexpr (MULTI) {
          if (am >= 0 && n < p.N)
            v += f16_bits_to_f32(static_cast<const uint16_t*>(ptrs[kMaxAdapters + am])[n]) * z;
        } else {
          if (n < p.N) v += f16_bits_to_f32(p.t.alpha[term][n]) * z;
        }
      }
    }
    if (owner && n < p.N && tt < p.T) store_out(p.y, p.y_dtype, tt * p.ldy + n, v, 0);
    __syncthreads();
  }
  // the ticket at the end: a wave's loads return in order, and one taken
  // right after the wait would hold up this wave's loads of the partials
  if (waited) lut::consumer_done(p.sync, lut::take_ticket(p.sync));
}

template <int TB, int KW>
__global__ void __launch_bounds__(kMainThreads) adapter_fused(lut::Stage1 s1, Main m, int n1) {
  extern __shared__ __align__(16) unsigned char smem[];
  if (static_cast<int>(blockIdx.x) < n1) {
    float* tbl = reinterpret_cast<float*>(smem);
    float* red = tbl + lut::tbl_elems<TB, KW, kMainWaves>();
    lut::stage1_role<float, TB, KW, lut::MODE_F, kMainWaves>(s1, blockIdx.x, tbl, red);
    lut::publish(m.sync, blockIdx.x);
    return;
  }
  main_role(m, static_cast<int64_t>(blockIdx.x) - n1, reinterpret_cast<float*>(smem));
}

// Several adapters, one per token, beside the one base: stage-1 workgroups
// hold one token each and run its adapter's B2 (or nothing for -1); the row
// workgroups stream W0 once for every token, then add each token's
// alpha . (B1 w) from its own adapter.
template <int KW>
__global__ void __launch_bounds__(kMainThreads) adapter_multi(lut::Stage1 s1, Main m,
                                                              lut::AdapterTable tab,
                                                              const int32_t* idx, int n1) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int bid = static_cast<int>(blockIdx.x);
  if (bid < n1) {
    // the workgroup's adapter, wave-uniform (so its pointers come from the
    // arguments by scalar loads)
    const int a = __builtin_amdgcn_readfirstlane(
        lut::token_adapter(idx, bid / (static_cast<int>(s1.nrt) * s1.ks), tab, m.sync, true));
    if (a >= 0) {
      float* tbl = reinterpret_cast<float*>(smem);
      float* red = tbl + lut::tbl_elems<1, KW, kMainWaves>();
      lut::stage1_role_src<float, 1, KW, lut::MODE_F, kMainWaves>(
          s1, lut::OneTerm{tab.b2[a], tab.gamma[a], tab.beta[a]}, bid, tbl, red);
    }
    lut::publish(m.sync, static_cast<unsigned>(bid));
    return;
  }
  // the adapters' B1 and alpha pointers in LDS (copied by constant index),
  // for the per-token reads of the row role
  const void** ptrs = reinterpret_cast<const void**>(
      smem + sizeof(float) * (kMainWaves * 16 * 16 + 16 * kRChunk));
  if (threadIdx.x == 0) {
#pragma unroll
    for (int q = 0; q < kMaxAdapters; ++q) {
      ptrs[q] = tab.b1[q];
      ptrs[kMaxAdapters + q] = tab.alpha[q];
    }
  }
  __syncthreads();
  main_role<true>(m, bid - n1, reinterpret_cast<float*>(smem), ptrs, tab.n, idx);
}

// ---- small ranks: every workgroup derives w itself ------------------------

constexpr int kSmallTiles = 4;  // 16-rank MFMA tiles, summed over the terms
constexpr int kSmallTerms = 2;  // more terms run out of registers
constexpr int kSteps = 4;       // 32-feature MFMA steps per group
constexpr int kGroup = kSteps * 32;  // one K-block of packed bits (kw = 4)
constexpr size_t kMaxLds = 160 * 1024;  // LDS of one workgroup

struct Small {
  const uint16_t* w0;
  int64_t ldw;
  TermPtrs t;
  int64_t N, M, R, T, ldx;
  const uint16_t* x;
  void* y;
  int y_dtype;
  int64_t ldy;
  int64_t kq;  // features per wave, a multiple of kGroup
  int fast;    // 16-byte W0 / x / B2 and 4-byte gamma loads allowed
};

// fp16 g as the exact sum hi + lo of two bf16 values: hi keeps the top eight
// significant bits, lo the last three (so both products with a bf16
// activation are exact in the fp32 accumulator).  Returns hi | lo << 16.
__device__ __forceinline__ uint32_t split_f16(uint16_t g) {
  const float f = f16_bits_to_f32(g);
  const uint32_t h = __float_as_uint(f) & 0xFFFF0000u;
  const uint32_t l = __float_as_uint(f - __uint_as_float(h));
  return (h >> 16) | (l & 0xFFFF0000u);
}

// 16 ranks x 16 tokens of (+-gamma) . x for the step whose B operand is bx:
// the lane's eight B2 bits pick sign masks from the table, which flip the
// split gamma of its eight features.
__device__ __forceinline__ floatx4 rank_step(floatx4 acc, uint32_t byte, const uint4& hi,
                                             const uint4& lo, const uint4& bx,
                                             const uint32_t* lut) {
  const uint4 m = *reinterpret_cast<const uint4*>(lut + 4 * byte);
  const uint4 ah = make_uint4(hi.x ^ m.x, hi.y ^ m.y, hi.z ^ m.z, hi.w ^ m.w);
  const uint4 alo = make_uint4(lo.x ^ m.x, lo.y ^ m.y, lo.z ^ m.z, lo.w ^ m.w);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ah),
                                                __builtin_bit_cast(bf16x8, bx), acc, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, alo),
                                                 __builtin_bit_cast(bf16x8, bx), acc, 0, 0, 0);
}

template <int L, int QR>
constexpr size_t small_lds_bytes() {
  constexpr size_t gam = size_t(kMainWaves) * L * 2 * kGroup * 2;
  constexpr size_t red = size_t(kMainWaves) * (L * QR + 1) * 256 * 4;
  return 4096 + (gam > red ? gam : red) + size_t(L * QR) * 256 * 4;
}

// Operands of one group (kSteps steps) of one wave, loaded one group ahead.
// Within a group, lane quarter lq takes features [32 lq, 32 lq + 32): step u
// gives it features 32 lq + 8 u .. + 8 (the MFMA sums over whichever features
// each lane holds, as long as A and B agree), so its B2 bits for the whole
// group are one word: byte u of word lq of the rank's 128-feature K-block.
template <int L, int QR>
struct Group {
  static constexpr int NQ = L * QR > 0 ? L * QR : 1;
  static constexpr int NL = L > 0 ? L : 1;
  uint4 a[kSteps], b[kSteps];  // W0 rows / x tokens, 8 features per lane
  uint32_t bw[NQ];             // B2 word lq of the lane's rank
  uint32_t g[NL];              // gamma of features 2 * lane, 2 * lane + 1
};

template <int L, int QR>
__device__ __forceinline__ void load_group(Group<L, QR>& G, const Small& p, int64_t k0,
                                           const uint16_t* wrow, const uint16_t* xrow,
                                           int lane, int li, int lq) {
#pragma unroll
  for (int term = 0; term < L; ++term)
    G.g[term] = *reinterpret_cast<const uint32_t*>(p.t.gamma[term] + k0 + 2 * lane);
#pragma unroll
  for (int q = 0; q < L * QR; ++q)
    G.bw[q] = p.t.b2[q / QR][((k0 >> 7) * 64 + 16 * (q % QR) + li) * 4 + lq];
#pragma unroll
  for (int u = 0; u < kSteps; ++u) {
    const int64_t k = k0 + lq * 32 + u * 8;
    G.a[u] = load16(wrow, k);
    G.b[u] = load16(xrow, k);
  }
}

template <int L, int QR>
__device__ __forceinline__ void compute_group(const Group<L, QR>& G, floatx4& acc,
                                              floatx4* wacc, uint16_t* mygam,
                                              const uint32_t* lut, int lane, int lq) {
  // the group's gamma, split, into the wave's own LDS slice (read back by
  // other lanes of the same wave only; the fences keep the order)
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
  for (int term = 0; term < L; ++term) {
    const uint32_t s0 = split_f16(G.g[term] & 0xFFFFu), s1 = split_f16(G.g[term] >> 16);
    reinterpret_cast<uint32_t*>(mygam + (term * 2) * kGroup)[lane] = (s0 & 0xFFFFu) | (s1 << 16);
    reinterpret_cast<uint32_t*>(mygam + (term * 2 + 1) * kGroup)[lane] =
        (s0 >> 16) | (s1 & 0xFFFF0000u);
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
  for (int u = 0; u < kSteps; ++u) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
        __builtin_bit_cast(bf16x8, G.a[u]), __builtin_bit_cast(bf16x8, G.b[u]), acc, 0, 0, 0);
#pragma unroll
    for (int term = 0; term < L; ++term) {
      const uint4 hi = *reinterpret_cast<const uint4*>(mygam + (term * 2) * kGroup + lq * 32 + u * 8);
      const uint4 lo =
          *reinterpret_cast<const uint4*>(mygam + (term * 2 + 1) * kGroup + lq * 32 + u * 8);
#pragma unroll
      for (int qr = 0; qr < QR; ++qr) {
        const int q = term * QR + qr;
        wacc[q] = rank_step(wacc[q], (G.bw[q] >> (8 * u)) & 0xFFu, hi, lo, G.b[u], lut);
      }
    }
    // keep the scheduler from hoisting every step's LDS reads (registers)
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Workgroup = 16 output rows.  Each wave streams its share of the features
// once per 16 tokens, one group ahead of its MFMAs, and feeds every x
// fragment to the base product and to the L * QR rank tiles.  LDS:
// sign-mask table [256][4] | per-wave split gamma [waves][L][hi, lo][kGroup]
// during the stream, reused afterwards for the per-wave partials
// [waves][1 + L * QR][16][16] | w [L * QR * 16][16].  L = 0 is the bare
// base product.
template <int L, int QR>
__global__ void __launch_bounds__(kMainThreads) adapter_small(Small p) {
  constexpr int NQ = L * QR;
  extern __shared__ __align__(16) unsigned char smem[];
  uint32_t* lut = reinterpret_cast<uint32_t*>(smem);
  uint16_t* gam = reinterpret_cast<uint16_t*>(smem + 4096);
  float* red = reinterpret_cast<float*>(smem + 4096);
  float* wfin = reinterpret_cast<float*>(smem + small_lds_bytes<L, QR>() - NQ * 256 * 4);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int li = lane & 15, lq = lane >> 4;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int64_t arow = n0 + li;
  const bool arow_ok = arow < p.N;
  const uint16_t* wrow = p.w0 + (arow_ok ? arow : 0) * p.ldw;
  const int64_t kbeg = wv * p.kq;
  const int64_t kend = min(p.M, kbeg + p.kq);
  const bool vec = p.fast != 0;
  const int64_t kwM = layout_kw(p.M), kwR = layout_kw(p.R);
  uint16_t* mygam = gam + wv * L * 2 * kGroup;
  // whole groups of this wave (the bounded steps take the rest)
  const int64_t ngroups = (vec && kend > kbeg) ? (kend - kbeg) / kGroup : 0;

  if (L > 0) {
    // dword d of entry b flips the low half where bit 2d of b is clear (-1)
    // and the high half where bit 2d + 1 is clear
    for (int e = tid; e < 1024; e += kMainThreads) {
      const uint32_t nb = ~static_cast<uint32_t>(e >> 2);
      const int d = e & 3;
      lut[e] = (((nb >> (2 * d)) & 1u) << 15) | (((nb >> (2 * d + 1)) & 1u) << 31);
    }
  }
  // owner threads (row oi, token oj) fetch their B1 row and alpha now
  const bool owner = tid < 256;
  const int oi = (tid >> 4) & 15, oj = tid & 15;
  const int64_t on = n0 + oi;
  uint32_t b1w[Group<L, QR>::NL][2];
  float al[Group<L, QR>::NL];
#pragma unroll
  for (int term = 0; term < L; ++term) {
    b1w[term][0] = b1w[term][1] = 0u;
    al[term] = 0.f;
    if (owner && on < p.N) {
      const uint32_t* b1 = p.t.b1[term] + ((on >> 6) * 64 + (on & 63)) * kwR;
      b1w[term][0] = b1[0];
      if (kwR > 1) b1w[term][1] = b1[1];
      al[term] = f16_bits_to_f32(p.t.alpha[term][on]);
    }
  }
  __syncthreads();

  for (int64_t tb0 = 0; tb0 < p.T; tb0 += 16) {
    const int64_t tok = tb0 + li;
    const bool tok_ok = tok < p.T;
    const uint16_t* xrow = p.x + (tok_ok ? tok : 0) * p.ldx;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    floatx4 wacc[Group<L, QR>::NQ];
#pragma unroll
    for (int q = 0; q < Group<L, QR>::NQ; ++q) wacc[q] = acc;
    // The stream runs one group ahead.  Each path either loads the next
    // group and then computes the current one, or computes the last one:
    // the loads in flight at every MFMA are then known to the compiler, which
    // otherwise waits for all of them (a load under a condition makes the
    // count unknown).  Two groups ahead (three buffers) measured no faster
    // and runs out of registers above one rank tile.
    if (ngroups > 0) {
      Group<L, QR> G0, G1;
      auto ld = [&](Group<L, QR>& G, int64_t g) {
        load_group(G, p, kbeg + g * kGroup, wrow, xrow, lane, li, lq);
      };
      auto cp = [&](const Group<L, QR>& G) { compute_group(G, acc, wacc, mygam, lut, lane, lq); };
      ld(G0, 0);
      for (int64_t g = 0;; g += 2) {  // G0 holds group g
        if (g + 1 >= ngroups) { cp(G0); break; }
        ld(G1, g + 1);
        cp(G0);
        if (g + 2 >= ngroups) { cp(G1); break; }
        ld(G0, g + 2);
        cp(G1);
      }
    }
    for (int64_t k0 = kbeg + ngroups * kGroup; k0 < kend; k0 += 32) {
      const int64_t k = k0 + lq * 8;
      const bool in = k < kend;
      const uint4 a = load8(wrow, k, kend, arow_ok && in, vec);
      const uint4 b = load8(xrow, k, kend, tok_ok && in, vec);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
      const int64_t kb = k0 / (32 * kwM), w = (k0 % (32 * kwM)) / 32;
#pragma unroll
      for (int term = 0; term < L; ++term) {
        uint32_t s[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          s[j] = (in && k + j < kend) ? split_f16(p.t.gamma[term][k + j]) : 0u;
        const uint4 hi = make_uint4((s[0] & 0xFFFFu) | (s[1] << 16), (s[2] & 0xFFFFu) | (s[3] << 16),
                                    (s[4] & 0xFFFFu) | (s[5] << 16), (s[6] & 0xFFFFu) | (s[7] << 16));
        const uint4 lo = make_uint4((s[0] >> 16) | (s[1] & 0xFFFF0000u), (s[2] >> 16) | (s[3] & 0xFFFF0000u),
                                    (s[4] >> 16) | (s[5] & 0xFFFF0000u), (s[6] >> 16) | (s[7] & 0xFFFF0000u));
#pragma unroll
        for (int qr = 0; qr < QR; ++qr) {
          const int64_t r = 16 * qr + li;
          const uint32_t word = p.t.b2[term][(kb * 64 + r) * kwM + w];
          const int q = term * QR + qr;
          wacc[q] = rank_step(wacc[q], (word >> (8 * lq)) & 0xFFu, hi, lo, b, lut);
        }
      }
    }
    __syncthreads();  // every wave is done with its gamma slice
    // D[i][j]: row (rank) i = 4 * (lane / 16) + r, token j = lane % 16
    float* myred = red + wv * (NQ + 1) * 256;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      myred[(4 * lq + r) * 16 + li] = acc[r];
#pragma unroll
      for (int q = 0; q < NQ; ++q) myred[(1 + q) * 256 + (4 * lq + r) * 16 + li] = wacc[q][r];
    }
    __syncthreads();
    // w = beta . (sum over the waves), as [tile * 16 + rank][token]
    for (int e = tid; e < NQ * 256; e += kMainThreads) {
      const int q = e >> 8, i = (e >> 4) & 15;
      float s = 0.f;
#pragma unroll
      for (int v = 0; v < kMainWaves; ++v) s += red[(v * (NQ + 1) + 1 + q) * 256 + (e & 255)];
      const int64_t r = 16 * (q % QR) + i;
      wfin[e] = r < p.R ? f16_bits_to_f32(p.t.beta[q / QR][r]) * s : 0.f;
    }
    float v = 0.f;
    if (owner) {
#pragma unroll
      for (int q = 0; q < kMainWaves; ++q) v += red[q * (NQ + 1) * 256 + tid];
    }
    __syncthreads();
    const int64_t tt = tb0 + oj;
    if (owner && on < p.N && tt < p.T) {
#pragma unroll
      for (int term = 0; term < L; ++term) {
        const float* wt = wfin + term * QR * 256 + oj;
        float z[4] = {0.f, 0.f, 0.f, 0.f};
        for (int r = 0; r < p.R; ++r) {
          const float wr = wt[r * 16];
          const uint32_t word = r < 32 ? b1w[term][0] : b1w[term][1];
          z[r & 3] += ((word >> (r & 31)) & 1u) ? wr : -wr;
        }
        v += al[term] * ((z[0] + z[1]) + (z[2] + z[3]));
      }
      store_out(p.y, p.y_dtype, tt * p.ldy + on, v, 0);
    }
    __syncthreads();
  }
}

// ---- small ranks, one token: stream waves and rank waves -----------------

// One-token decode is a stream of W0 (here 99.8% of the bytes) with a small
// matrix-core job beside it.  The two run in separate waves of the row
// workgroup so neither holds the other up:
// - 8 stream waves copy their share of the 16 W0 rows and of x global -> LDS
//   by DMA into a ring of S 128-feature groups each (no registers held by
//   loads in flight; a wave refills a slot as soon as it has read it) and
//   feed them to the base MFMA;
// - 4 rank waves copy x, gamma and the B2 words of a quarter of the
//   features into LDS first thing (a few tens of KiB, the same for every
//   workgroup, so L2 hits), split gamma exactly, and derive their quarter of
//   the unscaled w with adapter_small's arithmetic (exact split of gamma,
//   sign-mask table, fp32 MFMA sums) while the stream runs.
// The CU's memory pipeline serves its requests in order, so anything a wave
// loads while the stream is in flight waits behind several microseconds of
// W0; the rank inputs are therefore issued before the ring fills up, and
// nothing else is loaded until the stream ends.
constexpr int kRankWaves = 8;
constexpr int kTok1Threads = 64 * (kMainWaves + kRankWaves);

// Stream ring slot: the W0 fragments of a group [16 rows][16 chunks of
// 16 B] (16-byte position q of row r holds chunk q ^ r, so that the
// fragment reads of 16 rows hit 16 different bank groups) and x of the
// group (128 features).
constexpr int kTok1Slot = kSteps * 1024 + 256;
constexpr int kTok1Copies = kSteps + 1;  // DMA instructions per group
// Stream waves reading W0 into registers: loads of 512 features per row
// (M up to kVSFeatures)
constexpr int kVSLoads = 8;
constexpr int64_t kVSFeatures = 512 * kVSLoads;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// The rank inputs are copied in chunks of 4 groups (1 KiB of x, of gamma,
// and of the B2 words of each rank tile); chunk c goes to rank wave c % 8.
constexpr int kChunkGroups = 4;
constexpr int kTok1MaxChunks = 4;  // chunks per rank wave (M <= 16384)
__host__ __device__ inline int64_t tok1_padded_groups(int64_t M) {
  return (M / kGroup + kChunkGroups - 1) / kChunkGroups * kChunkGroups;
}

// LDS of adapter_tok1: sign-mask table [16 nibbles][32 copies][8 B] |
// stream ring [8][S][slot] | base partials [8][16] | rank inputs, over Gp = the groups
// rounded up to whole chunks: x [Gp * 128] (bf16, then the rank wave's
// scaled fp16), gamma [L][Gp * 128], B2 words [NQ][Gp][64] | rank partials
// [8][NQ * 16] | w [NQ * 16].
template <int L, int QR>
size_t tok1_lds_bytes(int S, int64_t M) {
  constexpr int NQ = L * QR;
  const int64_t Gp = tok1_padded_groups(M);
  return 4096 + size_t(kMainWaves) * S * kTok1Slot + size_t(kMainWaves) * 16 * 4 +
         size_t(Gp) * 256 + size_t(L) * Gp * 256 + size_t(NQ) * Gp * 256 +
         size_t(kRankWaves) * NQ * 16 * 4 + size_t(NQ) * 16 * 4;
}
// DMA instructions of one rank wave (at most 63 may be outstanding).
inline int64_t tok1_rank_copies(int L, int QR, int64_t M) {
  const int64_t nc = tok1_padded_groups(M) / kChunkGroups;
  return (nc + kRankWaves - 1) / kRankWaves * (1 + L + L * QR);
}

// Wait until every copy issued before the last `after` groups' copies (C
// per group) has landed: copies complete in issue order.
template <int C>
__device__ __forceinline__ void wait_groups(int after) {
  static_assert(2 * C < 64, "vmcnt range");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  if (after >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * C));
  else if (after == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(C));
  else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// T = 1, M a multiple of kGroup, 16-byte W0 / x / B2 and 4-byte gamma
// addresses, 1 or 2 terms and at most 4 rank tiles; LDS as tok1_lds_bytes.
template <int L, int QR, int S>
__global__ void __launch_bounds__(kTok1Threads) adapter_tok1(Small p) {
  constexpr int NQ = L * QR;
  constexpr int C = kTok1Copies;
  // S = 0: the stream waves read W0 into registers (M <= kVSFeatures), no ring
  constexpr bool VS = S == 0;
  static_assert(L >= 1 && S >= 0 && S <= 3, "terms, ring depth");
  extern __shared__ __align__(16) unsigned char smem[];
  const int64_t M = p.M, G = M / kGroup, Gp = tok1_padded_groups(M);
  const int64_t MP = Gp * kGroup;  // features of the padded rank inputs
  uint32_t* lut = reinterpret_cast<uint32_t*>(smem);
  unsigned char* ring = smem + 4096;
  float* red = reinterpret_cast<float*>(ring + size_t(kMainWaves) * S * kTok1Slot);  // [8][16]
  unsigned char* rx = reinterpret_cast<unsigned char*>(red + kMainWaves * 16);       // x
  unsigned char* rg = rx + 2 * MP;                                                   // gamma
  uint32_t* rb = reinterpret_cast<uint32_t*>(rg + size_t(L) * 2 * MP);               // B2 words
  float* pr = reinterpret_cast<float*>(rb + size_t(NQ) * Gp * 64);                   // [8][NQ*16]
  float* wfin = pr + kRankWaves * NQ * 16;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int li = lane & 15, lq = lane >> 4;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int64_t kwR = layout_kw(p.R);

  // the epilogue's operands, loaded by every wave before its copies (so
  // the waits for those cover them), unconditionally from in-bounds
  // addresses and masked where used: a load under a branch is waited for
  // at the branch's end
  const int oi = tid >> 4, oj = tid & 15;  // owners: row oi, rank lane oj
  const bool owner = tid < 256;
  const int64_t on = n0 + oi;
  const int64_t onc = min(on, p.N - 1);
  uint32_t b1w[L][2];
  uint16_t al[L];
#pragma unroll
  for (int term = 0; term < L; ++term) {
    const uint32_t* b1 = p.t.b1[term] + ((onc >> 6) * 64 + (onc & 63)) * kwR;
    b1w[term][0] = b1[0];
    b1w[term][1] = b1[kwR - 1];  // used only for ranks >= 32, where kw = 2
    al[term] = p.t.alpha[term][onc];
  }
  const int bq = min(tid >> 4, NQ - 1);
  const int64_t br = 16 * (bq % QR) + (tid & 15);
  const uint16_t bt = p.t.beta[bq / QR][min(br, p.R - 1)];

  // the stream waves' share of W0 and their ring (state of every wave;
  // used by waves 0-7)
  const int64_t kbeg = static_cast<int64_t>(wv) * p.kq;
  const int64_t kend = min(M, kbeg + p.kq);
  const int ng = kend > kbeg ? static_cast<int>((kend - kbeg) / kGroup) : 0;
  const uint16_t* wj[kSteps];  // W0 row 4j + lane / 16 (rows past N read row 0)
#pragma unroll
  for (int j = 0; j < kSteps; ++j) {
    const int64_t rw = n0 + 4 * j + (lane >> 4);
    wj[j] = p.w0 + (rw < p.N ? rw : 0) * p.ldw + 8 * ((lane & 15) ^ (4 * j + (lane >> 4)));
  }
  const unsigned ring0 = static_cast<unsigned>(reinterpret_cast<uintptr_t>(ring)) +
                         static_cast<unsigned>(wv * S * kTok1Slot);
  auto issue = [&](int g) {
    const unsigned sl = ring0 + static_cast<unsigned>((g % (S > 0 ? S : 1)) * kTok1Slot);
    const int64_t k0 = kbeg + static_cast<int64_t>(g) * kGroup;
#pragma unroll
    for (int j = 0; j < kSteps; ++j) copy16_to_lds(wj[j] + k0, sl + j * 1024);
    copy4_to_lds(p.x + k0 + 2 * lane, sl + kSteps * 1024);
  };
  const int pre = ng < S ? ng : S;

  // Order of issue: a CU serves its memory requests in order, so the rank
  // waves' inputs go ahead of most of the stream: the stream waves issue the
  // rest of their ring only after the barrier below.  With one rank tile the
  // rank work is short enough to start behind one group of W0 per stream
  // wave, which then starts the stream a barrier earlier (measured on 4096^2
  // rank 16, same box, four runs each: 10.05-10.43 -> 9.50-9.73 us; with
  // the whole ring ahead, 10.3-10.4; with two or more rank tiles even one
  // group ahead was level or slower).
  constexpr int kEarly = (!VS && NQ == 1) ? 1 : 0;
  if constexpr (kEarly > 0) {
    if (wv < kMainWaves)
      for (int g = 0; g < min(kEarly, pre); ++g) issue(g);
  }
  const int64_t nchunk = Gp / kChunkGroups;
  if (wv >= kMainWaves) {
    const unsigned rx0 = static_cast<unsigned>(reinterpret_cast<uintptr_t>(rx));
    const unsigned rg0 = static_cast<unsigned>(reinterpret_cast<uintptr_t>(rg));
    const unsigned rb0 = static_cast<unsigned>(reinterpret_cast<uintptr_t>(rb));
    // lane l copies 16 bytes of group 4c + l / 16 (past the last group it
    // reads the last group again, into the padding)
    for (int64_t c = wv - kMainWaves; c < nchunk; c += kRankWaves) {
      const int64_t gl = min(kChunkGroups * c + lane / 16, G - 1);
      const int64_t k = gl * kGroup + 8 * (lane & 15);
      const unsigned off = static_cast<unsigned>(c * kChunkGroups * 256);
      copy16_to_lds(p.x + k, rx0 + off);
#pragma unroll
      for (int term = 0; term < L; ++term)
        copy16_to_lds(p.t.gamma[term] + k, rg0 + static_cast<unsigned>(2 * MP * term) + off);
      // the 256 bytes of B2 words of ranks 16 (q % QR) .. + 15, per group
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        copy16_to_lds(p.t.b2[q / QR] + (gl * 64 + 16 * (q % QR)) * 4 + 4 * (lane & 15),
                      rb0 + static_cast<unsigned>(256 * q * Gp) + off);
    }
  }
  // sign masks by nibble: entry n (two dwords, four fp16 lanes) flips lane
  // h where bit h of n is clear; 32 interleaved copies, copy c of entry n
  // at 8-byte slot 32 n + c, so the 8-byte reads of 32 lanes (copy = lane
  // % 32) hit 32 different bank pairs whatever the nibbles
  for (int e = tid; e < 1024; e += kTok1Threads) {
    const uint32_t nb = ~static_cast<uint32_t>(e >> 6);
    const int d = e & 1;
    lut[e] = (((nb >> (2 * d)) & 1u) << 15) | (((nb >> (2 * d + 1)) & 1u) << 31);
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(lgkmcnt0_imm());
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);

  if (wv >= kMainWaves) {
    const int r = wv - kMainWaves;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    // x of the wave's chunks in fp16, scaled by sigma = a power of two that
    // puts their largest |x| in [2^14, 2^15): exact wherever the scaled
    // value is at least 2^-17 (x has 8 significant bits), so below 2^-31 of
    // the largest only; every product with gamma (fp16) is then exact in the
    // fp32 accumulator, and 1 / sigma is applied to the wave's partial
    // (each lane's 16 bytes of each chunk stay in registers between the
    // two passes: one LDS round trip, not two)
    uint4 xv[kTok1MaxChunks];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < kTok1MaxChunks; ++i) {
      const int64_t c = r + i * kRankWaves;
      xv[i] = c < nchunk ? reinterpret_cast<const uint4*>(rx + c * kChunkGroups * 256)[lane]
                         : make_uint4(0u, 0u, 0u, 0u);
      const uint32_t w4[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
#pragma unroll
      for (int h = 0; h < 4; ++h)
        amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(w4[h] << 16)),
                                 fabsf(__uint_as_float(w4[h] & 0xFFFF0000u))));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const float sig = act_scale(amax);
#pragma unroll
    for (int i = 0; i < kTok1MaxChunks; ++i) {
      const int64_t c = r + i * kRankWaves;
      if (c >= nchunk) break;
      const uint32_t w4[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
      uint32_t o[4];
#pragma unroll
      for (int h = 0; h < 4; ++h)
        o[h] = f32_to_f16_bits(sig * __uint_as_float(w4[h] << 16)) |
               (static_cast<uint32_t>(f32_to_f16_bits(sig * __uint_as_float(w4[h] & 0xFFFF0000u))) << 16);
      reinterpret_cast<uint4*>(rx + c * kChunkGroups * 256)[lane] = make_uint4(o[0], o[1], o[2], o[3]);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    floatx4 wacc[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) wacc[q] = floatx4{0.f, 0.f, 0.f, 0.f};
    // Each step's operands come from LDS (x', gamma, and a sign mask per
    // rank tile picked by the lane's B2 byte); they are read one step
    // ahead of the MFMAs that use them, so a step's LDS round trip overlaps
    // the previous step's work (read just in time, every tile waited for
    // its own round trip).
    struct StepOps {
      uint4 x, g[L], m[NQ];
    };
    const uint32_t* mylut = lut + 2 * (lane & 31);
    for (int64_t c = r; c < nchunk; c += kRankWaves)
    for (int64_t g = c * kChunkGroups; g < min(G, (c + 1) * kChunkGroups); ++g) {
      uint32_t bw[NQ];
#pragma unroll
      for (int q = 0; q < NQ; ++q) bw[q] = rb[(q * Gp + g) * 64 + 4 * li + lq];
      auto load_step = [&](int u, StepOps& o) {
        const int64_t k = g * kGroup + lq * 32 + u * 8;
        o.x = *reinterpret_cast<const uint4*>(rx + 2 * k);
#pragma unroll
        for (int term = 0; term < L; ++term)
          o.g[term] = *reinterpret_cast<const uint4*>(rg + 2 * MP * term + 2 * k);
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          const uint32_t byte = bw[q] >> (8 * u);
          const uint2 lo = *reinterpret_cast<const uint2*>(mylut + 64 * (byte & 15u));
          const uint2 hi = *reinterpret_cast<const uint2*>(mylut + 64 * ((byte >> 4) & 15u));
          o.m[q] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
      };
      StepOps cur, nxt;
      load_step(0, cur);
#pragma unroll
      for (int u = 0; u < kSteps; ++u) {
        if (u + 1 < kSteps) load_step(u + 1, nxt);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          // 16 ranks x 16 tokens of (+-gamma) . x': the mask flips the signs
          // of the lane's eight gammas where its B2 bits are 0
          const uint4& g4 = cur.g[q / QR];
          const uint4 a = make_uint4(g4.x ^ cur.m[q].x, g4.y ^ cur.m[q].y, g4.z ^ cur.m[q].z,
                                     g4.w ^ cur.m[q].w);
          wacc[q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                           __builtin_bit_cast(f16x8, cur.x), wacc[q], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (u + 1 < kSteps) cur = nxt;
      }
    }
    const float isig = 1.f / sig;  // exact: sig is a power of two
    // D[i][j]: rank i = 4 * (lane / 16) + r, token j = lane % 16; the token
    // is column 0
    if (li == 0) {
#pragma unroll
      for (int q = 0; q < NQ; ++q)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) pr[(r * NQ + q) * 16 + 4 * lq + rr] = wacc[q][rr] * isig;
    }
  } else if constexpr (VS) {
    // ---- stream role, registers: rows 2 wv and 2 wv + 1 of the 16 ------
    // Each load of a wave reads 1 KiB of one row (512 features, 16 bytes a
    // lane, consecutive lanes consecutive), as a plain streaming read does;
    // x of the same features is held in registers, and the row's dot
    // product is summed over the lanes at the end.  Every load is issued
    // from an in-bounds address (features past M and rows past N read
    // feature 0 / row 0) and masked where it is used.
    const int nl = static_cast<int>((M + 511) / 512);
    uint4 xr[kVSLoads], wr[2][kVSLoads];
    const uint16_t* wrow[2];
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int64_t rw = n0 + 2 * wv + rr;
      wrow[rr] = p.w0 + (rw < p.N ? rw : 0) * p.ldw;
    }
#pragma unroll
    for (int j = 0; j < kVSLoads; ++j) {
      const int64_t k = 512 * j + 8 * lane;
      const int64_t kc = j < nl && k < M ? k : 0;
      xr[j] = *reinterpret_cast<const uint4*>(p.x + kc);
    }
#pragma unroll
    for (int rr = 0; rr < 2; ++rr)
#pragma unroll
      for (int j = 0; j < kVSLoads; ++j) {
        const int64_t k = 512 * j + 8 * lane;
        const int64_t kc = j < nl && k < M ? k : 0;
        wr[rr][j] = *reinterpret_cast<const uint4*>(wrow[rr] + kc);
      }
    float sr[2] = {0.f, 0.f};
#pragma unroll
    for (int rr = 0; rr < 2; ++rr)
#pragma unroll
      for (int j = 0; j < kVSLoads; ++j) {
        const bool in = j < nl && 512 * j + 8 * lane < M;
        const uint4 w = wr[rr][j], xv = xr[j];
        const uint32_t wa[4] = {w.x, w.y, w.z, w.w}, xa[4] = {xv.x, xv.y, xv.z, xv.w};
        float d = 0.f;
#pragma unroll
        for (int h = 0; h < 4; ++h)
          d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wa[h]),
                                              __builtin_bit_cast(bf16x2, xa[h]), d, false);
        sr[rr] += in ? d : 0.f;
      }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      sr[0] += __shfl_xor(sr[0], off);
      sr[1] += __shfl_xor(sr[1], off);
    }
    if (lane < 16) red[wv * 16 + lane] = lane == 2 * wv ? sr[0] : (lane == 2 * wv + 1 ? sr[1] : 0.f);
  } else {
    // ---- stream role: the wave's share of W0 through the ring ----------
    for (int g = min(kEarly, pre); g < pre; ++g) issue(g);
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int g = 0; g < ng; ++g) {
      wait_groups<C>(min(S - 1, ng - 1 - g));  // the groups issued after g
      const unsigned char* sl = ring + (wv * S + g % S) * kTok1Slot;
#pragma unroll
      for (int u = 0; u < kSteps; ++u) {
        const uint4 a = *reinterpret_cast<const uint4*>(sl + 16 * (16 * li + ((4 * lq + u) ^ li)));
        const uint4 xb = *reinterpret_cast<const uint4*>(sl + kSteps * 1024 + lq * 64 + u * 16);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                      __builtin_bit_cast(bf16x8, xb), acc, 0, 0, 0);
      }
      if (g + S < ng) {
        // this wave's reads of the slot are complete before it is refilled
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(lgkmcnt0_imm());
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        issue(g + S);
      }
    }
    if (li == 0) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) red[wv * 16 + 4 * lq + rr] = acc[rr];
    }
  }
  __syncthreads();
  // w = beta . (sum over the rank waves in order)
  if (tid < NQ * 16) {
    float sum = 0.f;
#pragma unroll
    for (int r = 0; r < kRankWaves; ++r) sum += pr[r * NQ * 16 + tid];
    wfin[tid] = br < p.R ? f16_bits_to_f32(bt) * sum : 0.f;
  }
  __syncthreads();
  if (owner) {
    // lane oj of row oi takes ranks oj, oj + 16, ...; 16 lanes per row
    float v = 0.f;
#pragma unroll
    for (int term = 0; term < L; ++term) {
      float z = 0.f;
#pragma unroll
      for (int qr = 0; qr < QR; ++qr) {
        const int rk = 16 * qr + oj;
        const float wr = wfin[term * QR * 16 + rk];
        const uint32_t word = rk < 32 ? b1w[term][0] : b1w[term][1];
        z += ((word >> (rk & 31)) & 1u) ? wr : -wr;
      }
      v += f16_bits_to_f32(al[term]) * z;
    }
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) v += __shfl_xor(v, off);
    if (oj == 0 && on < p.N) {
      float base = 0.f;
#pragma unroll
      for (int q = 0; q < kMainWaves; ++q) base += red[q * 16 + oi];
      store_out(p.y, p.y_dtype, on, base + v, 0);
    }
  }
}

}  // namespace

hipError_t launch_multi_adapter(const uint16_t* w0, int64_t ldw, const TermPtrs* adapters,
                                int n_adapters, int64_t N, int64_t M, int64_t R,
                                const int32_t* idx, const void* x, int64_t T, int64_t ldx,
                                void* y, int y_dtype, int64_t ldy, void* ws, hipStream_t s) {
  lut::AdapterTable tab{};
  tab.n = n_adapters;
  for (int a = 0; a < n_adapters; ++a) {
    tab.b1[a] = adapters[a].b1[0];
    tab.b2[a] = adapters[a].b2[0];
    tab.alpha[a] = adapters[a].alpha[0];
    tab.beta[a] = adapters[a].beta[0];
    tab.gamma[a] = adapters[a].gamma[0];
  }
  Main m{};
  m.w0 = w0; m.ldw = ldw; m.N = N; m.M = M; m.R = R; m.T = T;
  m.ldx = ldx; m.x = static_cast<const uint16_t*>(x); m.y = y;
  m.y_dtype = y_dtype; m.ldy = ldy;
  m.kq = ((M + kMainWaves - 1) / kMainWaves + 31) / 32 * 32;
  m.vec = (ldw % 8 == 0) && (ldx % 8 == 0) &&
          (reinterpret_cast<uintptr_t>(w0) % 16 == 0) &&
          (reinterpret_cast<uintptr_t>(x) % 16 == 0);
  m.nmain = static_cast<unsigned>((N + 15) / 16);
  // stage 1 in one-token blocks (each token its own adapter)
  int n1 = 0;
  lut::Stage1 a = make_stage1(adapters[0], M, R, x, DBF_BF16, T, ldx, ws, true, &n1, kMainWaves);
  int64_t per = 0;
  a.ntb = static_cast<int>(T);
  for (int q = 0; q < n_adapters; ++q)  // 8-byte gamma loads for every adapter
    if (reinterpret_cast<uintptr_t>(adapters[q].gamma[0]) % 8 != 0) a.vec4 = 0;
  a.ks = lut::pick_ks(a.nrt * T, 1, a.nkb, 512, &per, kMainWaves);
  a.kb_per_split = per;
  n1 = static_cast<int>(a.nrt * a.ks * T);
  m.ws = static_cast<const float*>(a.ws);
  m.ks = a.ks;
  m.rs = a.rs;
  m.sync = lut::make_sync(ws, n1, m.nmain);
  const size_t main_lds = sizeof(float) * (kMainWaves * 16 * 16 + 16 * kRChunk) +
                          2 * kMaxAdapters * sizeof(void*);
  const int kw = static_cast<int>(layout_kw(M));
  const dim3 grid(static_cast<unsigned>(n1) + m.nmain);
#define DBF_MA(KW_) \
  adapter_multi<KW_><<<grid, kMainThreads, std::max(main_lds, lut::lds_bytes<float, 1, KW_, kMainWaves>()), s>>>(a, m, tab, idx, n1)
  switch (kw) {
    case 1: DBF_MA(1); break;
    case 2: DBF_MA(2); break;
    case 3: DBF_MA(3); break;
    default: DBF_MA(4); break;
  }
#undef DBF_MA
  return hipGetLastError();
}

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
  const int64_t qr = t.n > 0 ? (R + 15) / 16 : 0;
  if (t.n <= kSmallTerms && t.n * qr <= kSmallTiles) {
    Small sp{};
    sp.w0 = w0; sp.ldw = ldw; sp.t = t; sp.N = N; sp.M = M; sp.R = R; sp.T = T;
    sp.ldx = ldx; sp.x = m.x; sp.y = y; sp.y_dtype = y_dtype; sp.ldy = ldy;
    sp.kq = ((M + kMainWaves - 1) / kMainWaves + kGroup - 1) / kGroup * kGroup;
    sp.fast = m.vec;
    for (int i = 0; i < t.n; ++i)
      if (reinterpret_cast<uintptr_t>(t.b2[i]) % 16 != 0 ||
          reinterpret_cast<uintptr_t>(t.gamma[i]) % 4 != 0)
        sp.fast = 0;
    // LDS above 64 KiB needs the kernel's attribute raised once (to the
    // whole budget: the one-token kernel's LDS depends on M)
    auto go = [&](auto kern, size_t lds, int threads) -> hipError_t {
      static bool attr_set = false;  // per instantiation; idempotent if raced
      if (!attr_set) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 static_cast<int>(kMaxLds));
        if (e != hipSuccess) return e;
        attr_set = true;
      }
      kern<<<dim3(m.nmain), threads, lds, s>>>(sp);
      return hipGetLastError();
    };
    // one token on whole 128-feature groups (16-byte gamma, since it is
    // copied 16 bytes at a time), when the rank inputs fit in LDS beside a
    // ring of at least 2 groups per stream wave.  With four rank tiles the
    // stream waves read W0 into registers instead (no ring; M <= 4096):
    // there the rank waves bound the call, and they no longer share the
    // LDS with the ring's copies and reads (measured on 4096^2, one token:
    // rank 64 10.86 -> 10.19 us; rank 16 9.42 -> 9.67, rank 32 and 48
    // level, so those keep the ring)
    bool tok1 = T == 1 && sp.fast && M % kGroup == 0 && t.n > 0 &&
                tok1_padded_groups(M) / kChunkGroups <= kRankWaves * kTok1MaxChunks &&
                tok1_rank_copies(t.n, static_cast<int>(qr), M) <= 63;
    for (int i = 0; i < t.n; ++i)
      if (reinterpret_cast<uintptr_t>(t.gamma[i]) % 16 != 0) tok1 = false;
#define DBF_SM(L_, QR_)                                                                     \
  if constexpr (L_ > 0) {                                                                   \
    if (tok1 && L_ * QR_ >= 4 && M <= kVSFeatures && tok1_lds_bytes<L_, QR_>(0, M) <= kMaxLds) \
      return go(adapter_tok1<L_, QR_, 0>, tok1_lds_bytes<L_, QR_>(0, M), kTok1Threads);     \
    if (tok1 && tok1_lds_bytes<L_, QR_>(3, M) <= kMaxLds)                                   \
      return go(adapter_tok1<L_, QR_, 3>, tok1_lds_bytes<L_, QR_>(3, M), kTok1Threads);     \
    if (tok1 && tok1_lds_bytes<L_, QR_>(2, M) <= kMaxLds)                                   \
      return go(adapter_tok1<L_, QR_, 2>, tok1_lds_bytes<L_, QR_>(2, M), kTok1Threads);     \
  }                                                                                         \
  return go(adapter_small<L_, QR_>, small_lds_bytes<L_, QR_>(), kMainThreads)
    switch (t.n * 4 + static_cast<int>(qr)) {
      case 0: DBF_SM(0, 1);
      case 5: DBF_SM(1, 1);
      case 6: DBF_SM(1, 2);
      case 7: DBF_SM(1, 3);
      case 8: DBF_SM(1, 4);
      case 9: DBF_SM(2, 1);
      default: DBF_SM(2, 2);
    }
#undef DBF_SM
  }
  const size_t main_lds = sizeof(float) * (kMainWaves * 16 * 16 + 16 * kRChunk);
  int n1 = 0;
  const lut::Stage1 a = make_stage1(t, M, R, x, DBF_BF16, T, ldx, ws, true, &n1, kMainWaves);
  m.ws = static_cast<const float*>(a.ws);
  m.ks = a.ks;
  m.rs = a.rs;
  m.sync = lut::make_sync(ws, n1, m.nmain);
  const int tb = lut::pick_tb(T), kw = static_cast<int>(layout_kw(M));
  const dim3 grid(static_cast<unsigned>(n1) + m.nmain);
#define DBF_AD(TB_, KW_)                                                                 \
  adapter_fused<TB_, KW_><<<grid, kMainThreads, std::max(main_lds, lut::lds_bytes<float, TB_, KW_, kMainWaves>()), \
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
