// MFMA path of the double-binary layer (large token counts): the two
// sign-accumulate products of LoRDBA section 2 ("Kernel de Inferencia") /
// DBF section 2 ("Inferencia") as two tiled products on the matrix cores,
// with the +-1 signs unpacked from the packed bits straight into MFMA
// operand registers (exact in fp16).
//
//   prep:     u_i = fp16(sigma_t gamma_i . x) for every term, sigma_t the
//             power of two that puts the token's largest |gamma_i . x| (over
//             every term) in [2^14, 2^15); per token l_i[t] = sum_m
//             |u_i[t, m]| / sigma_t; bmax_i = max_r |beta_i[r]|
//   scale:    s_t = 2^e, the largest power of two with
//             s_t * max_i(bmax_i * l_i[t]) * (1 + 2^-8) <= 2^14; since
//             |w_i[t, r]| <= bmax_i * l_i[t], every s_t * w fits fp16
//   stage 1:  v_i[t, r] = fp16(s_t / sigma_t * beta_i[r] * sum_m S2_i[r, m] u_i[t, m])
//   stage 2:  y[t, n] = (1 / s_t) sum_i sum_r (+-alpha_i[n]) v_i[t, r]
//             (one term: alpha_1[n] / s_t * sum_r (+-1) v_1[t, r], alpha
//             applied in the epilogue)
//
// Rounding: u and v are each rounded to fp16 once (relative 2^-11), all
// sums are fp32; alpha, beta and the +-1 signs are exact in fp16.  Both
// fp16 intermediates carry a per-token power of two, so any finite input
// that gives a finite output stays inside the fp16 range.
//
// Operand order.  The MFMA sums over k, so any k order works as long as A
// and B agree.  u and v are stored with each 32 features reordered as pairs
// (k, k + 16): position 2j holds k = j, position 2j + 1 holds k = j + 16.
// A lane then builds its B fragment for pairs (k, k + 16) from one 32-bit
// word of its packed sign row with one shift and one bit merge per pair
// (v_and_or_b32 in stage 1, where the magnitude is the constant 1;
// v_bfi_b32 in stage 2): bits k and k + 16 land on the two fp16 sign bits.  With several terms,
// stage 2 folds alpha into those values (+-|alpha_n|, exact), so all terms
// accumulate into the same registers.
//
// Tiles: a workgroup computes BM tokens x BN columns with 4 wavefronts, each
// owning BN / 4 columns of all BM tokens with v_mfma_f32_32x32x16_f16.  K
// advances 128 features (one K-block of the bit layout) per step; the fp16
// activation tile (A) and the columns' sign words are copied global -> LDS
// directly (two stages, one step ahead), the A rows XOR-swizzled for
// conflict-free ds_read_b128 fragments.  Workgroup indices are remapped so
// that consecutive tiles of one XCD share token rows (L2 reuse).  The tile
// shape is chosen per launch so that at least ~256 workgroups run; with
// fewer tiles than that (tens of tokens) K is split over the grid's z
// dimension, each split writes an fp32 partial tile, and reduce1_kernel /
// reduce2_kernel sum the splits in order and apply the scales.
#include <algorithm>
#include <type_traits>

#include "dbf_internal.h"

namespace dbf {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int BK = 128;      // features per K step (one K-block of the bit layout)
constexpr int kThreads = 256;
constexpr int kStages = 2;   // LDS stages of the K-step pipeline

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ inline int64_t kpad(int64_t K) { return (K + BK - 1) / BK * BK; }

// Power-of-two scale of the fp16 intermediate from the bound b = max_i
// bmax_i * l_i[t]: s * b * (1 + 2^-8) <= 2^14.  The exponent is clamped so
// that s and 1 / s stay finite fp32 normals.
__device__ __forceinline__ float scale_from_bound(float b) {
  if (!(b > 0.f)) return 1.f;
  int e = 0;
  frexpf(b * (1.f + 1.f / 256.f), &e);  // b' = f * 2^e, f in [0.5, 1)
  return ldexpf(1.f, max(-100, min(100, 14 - e)));
}

// The largest bmax_i * l1_i[tok] over the terms.  Every term slot is loaded
// (slots past L repeat the last term, which leaves the maximum unchanged), so
// no load waits behind a loop branch.
__device__ __forceinline__ float term_bound(const float* bmax, const float* l1, int L, int64_t T,
                                            int64_t tok) {
  float b[DBF_MAX_TERMS], l[DBF_MAX_TERMS];
#pragma unroll
  for (int i = 0; i < DBF_MAX_TERMS; ++i) {
    const int ii = min(i, L - 1);
    b[i] = bmax[ii];
    l[i] = l1[static_cast<int64_t>(ii) * T + tok];
  }
  float bnd = 0.f;
#pragma unroll
  for (int i = 0; i < DBF_MAX_TERMS; ++i) bnd = fmaxf(bnd, b[i] * l[i]);
  return bnd;
}

// ---- prep: u = fp16(sigma_t gamma . x) in pair order, l1 norms, max |beta|
//
// sigma_t (act_scale of the token's largest |gamma_i . x| over every term) is
// common to the terms of a token, so their products still add in one
// accumulator; it is written to sig[t] and divided out after the products.
// l1[i][t] is sum_m |u_i[t, m]| / sigma_t, the norm at the true scale.
struct PrepArgs {
  const void* x;
  int x_dtype;
  int64_t ldx, T, M, mpad, R;
  int L;
  const uint16_t* gamma[DBF_MAX_TERMS];
  const uint16_t* beta[DBF_MAX_TERMS];
  _Float16* u;  // [L][T][mpad]
  float* l1;    // [L][T]
  float* bmax;  // [L]
  float* sig;   // [T]
  int vec;      // 16-byte loads of x and gamma allowed (2: x is fp32)
};

constexpr int kPrepSeg = 8192;  // features of a row staged in LDS at a time
constexpr int kPrepRound = 4;   // 16-byte chunks a thread loads at once

// gamma . x of the chunks cs + 256 j (j < kPrepRound) of 8 features each
// (chunk c holds features 8 c .. 8 c + 7 of the row), zeros past M.  The
// vector loads of whole chunks are issued together with their addresses
// clamped to the last whole chunk, so no load sits under a branch; the one
// chunk that straddles M is read element by element.
__device__ __forceinline__ void prep_round(const PrepArgs& p, int term, int64_t tok, int64_t cs,
                                           float (&a)[kPrepRound][8]) {
  const uint16_t* g = p.gamma[term];
  const int64_t nfull = p.M / 8;
  if (p.vec != 0 && nfull > 0) {
    uint4 xv[kPrepRound][2], gv[kPrepRound];
#pragma unroll
    for (int j = 0; j < kPrepRound; ++j) {
      const int64_t k0 = 8 * min(cs + 256 * j, nfull - 1);
      if (p.vec == 2) {
        const float* xf32 = static_cast<const float*>(p.x) + tok * p.ldx + k0;
        xv[j][0] = *reinterpret_cast<const uint4*>(xf32);
        xv[j][1] = *reinterpret_cast<const uint4*>(xf32 + 4);
      } else {
        xv[j][0] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.x) + tok * p.ldx + k0);
      }
      gv[j] = *reinterpret_cast<const uint4*>(g + k0);
    }
#pragma unroll
    for (int j = 0; j < kPrepRound; ++j) {
      const int64_t c = cs + 256 * j;
      if (c < nfull) {
        const uint32_t gw[4] = {gv[j].x, gv[j].y, gv[j].z, gv[j].w};
        if (p.vec == 2) {
          const uint32_t xw[8] = {xv[j][0].x, xv[j][0].y, xv[j][0].z, xv[j][0].w,
                                  xv[j][1].x, xv[j][1].y, xv[j][1].z, xv[j][1].w};
#pragma unroll
          for (int i = 0; i < 8; ++i)
            a[j][i] = f16_bits_to_f32(static_cast<uint16_t>(gw[i >> 1] >> (16 * (i & 1)))) *
                      __uint_as_float(xw[i]);
        } else {
          const uint32_t xw[4] = {xv[j][0].x, xv[j][0].y, xv[j][0].z, xv[j][0].w};
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint16_t xb = static_cast<uint16_t>(xw[i >> 1] >> (16 * (i & 1)));
            const uint16_t gb = static_cast<uint16_t>(gw[i >> 1] >> (16 * (i & 1)));
            const float xf = p.x_dtype == DBF_BF16 ? bf16_bits_to_f32(xb) : f16_bits_to_f32(xb);
            a[j][i] = f16_bits_to_f32(gb) * xf;
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int64_t k = 8 * c + i;
          a[j][i] = k < p.M ? f16_bits_to_f32(g[k]) * load_act(p.x, p.x_dtype, tok * p.ldx + k) : 0.f;
        }
      }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < kPrepRound; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t k = 8 * (cs + 256 * j) + i;
      a[j][i] = k < p.M ? f16_bits_to_f32(g[k]) * load_act(p.x, p.x_dtype, tok * p.ldx + k) : 0.f;
    }
}

// Sum (or max) of v over the 256 threads, returned to every thread.
__device__ __forceinline__ float block_reduce(float v, bool sum, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float o = __shfl_xor(v, off);
    v = sum ? v + o : fmaxf(v, o);
  }
  __syncthreads();  // red may still be read from an earlier call
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) r = sum ? r + red[w] : fmaxf(r, red[w]);
  return r;
}

// Feature e of a 16-byte chunk of x as loaded: 8 fp32 values in x0, x1
// (X32) or 8 fp16 / bf16 values in x0.
template <bool X32>
__device__ __forceinline__ float chunk_x(const PrepArgs& p, const uint4& x0, const uint4& x1, int e) {
  if constexpr (X32) {
    const uint32_t w[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    return __uint_as_float(w[e]);
  }
  const uint32_t w[4] = {x0.x, x0.y, x0.z, x0.w};
  const uint16_t b = static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1)));
  return p.x_dtype == DBF_BF16 ? bf16_bits_to_f32(b) : f16_bits_to_f32(b);
}
__device__ __forceinline__ float chunk_g(const uint4& g, int e) {
  const uint32_t w[4] = {g.x, g.y, g.z, g.w};
  return f16_bits_to_f32(static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1))));
}

// Term slots whose gamma rows the fast path of prep_kernel loads per round
// trip: 0 = the workgroup's own term only (one term), else 2 or 4.  X32: x
// is fp32 read with 16-byte loads (vec == 2).  Both are template parameters
// so that no load of the fast path sits under a branch.
template <int LG, bool X32>
__global__ void __launch_bounds__(256) prep_kernel(PrepArgs p) {
  __shared__ float red[4];
  __shared__ __align__(16) _Float16 useg[kPrepSeg];
  const int tid = threadIdx.x;
  const int64_t blk = blockIdx.x;
  // the L max|beta| workgroups come first, so that they start early
  if (blk < p.L) {
    const int term = static_cast<int>(blk);
    const uint16_t* bt = p.beta[term];
    float m = 0.f;
    if (p.R > 0) {
      // 16 loads in flight per thread; indices past R repeat the last value
      constexpr int kU = 16;
      for (int64_t r0 = 0; r0 < p.R; r0 += 256 * kU) {
        uint16_t b[kU];
#pragma unroll
        for (int k = 0; k < kU; ++k) b[k] = bt[min<int64_t>(r0 + 256 * k + tid, p.R - 1)];
#pragma unroll
        for (int k = 0; k < kU; ++k) m = fmaxf(m, fabsf(f16_bits_to_f32(b[k])));
      }
    }
    m = block_reduce(m, false, red);
    if (tid == 0) p.bmax[term] = m;
    return;
  }
  const int64_t row = blk - p.L;  // term * T + token
  const int term = static_cast<int>(row / p.T);
  const int64_t tok = row - static_cast<int64_t>(term) * p.T;
  const int64_t nch = p.mpad / 8;  // chunks of the padded row
  constexpr int64_t kRoundCh = 256 * kPrepRound;
  // one round covers this thread's whole row: its values stay in registers
  // from the max pass to the conversion (the max pass takes the terms in
  // the order term + 1, ..., term, so the last one is this workgroup's own)
  const bool single = nch <= kRoundCh && p.mpad <= kPrepSeg;
  float keep[kPrepRound][8];

  // pass 1: the token's largest |gamma_i . x| over every term
  float amx = 0.f;
  if (single && p.vec == (X32 ? 2 : 1) && p.M % 8 == 0) {
    // Fast path: every chunk is whole or past M.  max_i |gamma_i[m] x[m]|
    // = |x[m]| max_i |gamma_i[m]| holds for the rounded products too
    // (rounding is monotonic; fmaxf skips a NaN gamma like the per-term
    // maximum does), so x and the own term's gamma are loaded once and the
    // terms' gamma rows LG at a time, each group in one round trip.
    const int64_t nfull = p.M / 8;
    const uint16_t* gown = p.gamma[term];
    uint4 xr[kPrepRound][2], gr[kPrepRound];
    int64_t k0[kPrepRound];
#pragma unroll
    for (int j = 0; j < kPrepRound; ++j) {
      k0[j] = 8 * min(tid + 256 * j, nfull - 1);
      if constexpr (X32) {
        const float* xf32 = static_cast<const float*>(p.x) + tok * p.ldx + k0[j];
        xr[j][0] = *reinterpret_cast<const uint4*>(xf32);
        xr[j][1] = *reinterpret_cast<const uint4*>(xf32 + 4);
      } else {
        xr[j][0] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.x) + tok * p.ldx + k0[j]);
        xr[j][1] = make_uint4(0u, 0u, 0u, 0u);  // unused
      }
      gr[j] = *reinterpret_cast<const uint4*>(gown + k0[j]);
    }
    // the own term's gamma is folded in last: no use of it stands between
    // its loads and those of the first group
    float gm[kPrepRound][8];
#pragma unroll
    for (int j = 0; j < kPrepRound; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) gm[j][e] = 0.f;
    if constexpr (LG > 0) {
      for (int g0 = 0; g0 < p.L; g0 += LG) {
        uint4 gs[LG][kPrepRound];
#pragma unroll
        for (int i = 0; i < LG; ++i) {
          const uint16_t* gi = p.gamma[min(g0 + i, p.L - 1)];
#pragma unroll
          for (int j = 0; j < kPrepRound; ++j) gs[i][j] = *reinterpret_cast<const uint4*>(gi + k0[j]);
        }
#pragma unroll
        for (int i = 0; i < LG; ++i)
#pragma unroll
          for (int j = 0; j < kPrepRound; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) gm[j][e] = fmaxf(gm[j][e], fabsf(chunk_g(gs[i][j], e)));
      }
    }
#pragma unroll
    for (int j = 0; j < kPrepRound; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) gm[j][e] = fmaxf(gm[j][e], fabsf(chunk_g(gr[j], e)));
#pragma unroll
    for (int j = 0; j < kPrepRound; ++j) {
      const bool live = tid + 256 * j < nfull;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float xv = chunk_x<X32>(p, xr[j][0], xr[j][1], e);
        keep[j][e] = live ? chunk_g(gr[j], e) * xv : 0.f;
        if (live) amx = fmaxf(amx, gm[j][e] * fabsf(xv));
      }
    }
  } else {
    for (int ii = 0; ii < p.L; ++ii) {
      const int i = (term + 1 + ii) % p.L;
      for (int64_t cs = tid; cs < nch; cs += kRoundCh) {
        prep_round(p, i, tok, cs, keep);
#pragma unroll
        for (int j = 0; j < kPrepRound; ++j)
#pragma unroll
          for (int e = 0; e < 8; ++e) amx = fmaxf(amx, fabsf(keep[j][e]));
      }
    }
  }
  const float sig = act_scale(block_reduce(amx, false, red));
  if (term == 0 && tid == 0) p.sig[tok] = sig;

  // pass 2: u = fp16(sigma . gamma . x) in natural order into LDS, a segment
  // of kPrepSeg features at a time, then each thread writes one 16-byte
  // chunk of the pair order (positions 2 j and 2 j + 1 hold features j and
  // j + 16 of a 32-feature group)
  float acc = 0.f;
  _Float16* out = p.u + row * p.mpad;
  for (int64_t seg = 0; seg < p.mpad; seg += kPrepSeg) {
    const int64_t segn = min<int64_t>(kPrepSeg, p.mpad - seg);
    const int64_t c0 = seg / 8, c1 = c0 + segn / 8;
    for (int64_t cs = c0 + tid; cs < c1; cs += kRoundCh) {
      if (!single) prep_round(p, term, tok, cs, keep);
#pragma unroll
      for (int j = 0; j < kPrepRound; ++j) {
        const int64_t c = cs + 256 * j;
        if (c >= c1) break;
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const _Float16 lo = static_cast<_Float16>(sig * keep[j][2 * q]);
          const _Float16 hi = static_cast<_Float16>(sig * keep[j][2 * q + 1]);
          acc += fabsf(static_cast<float>(lo)) + fabsf(static_cast<float>(hi));
          o[q] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) |
                 (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) << 16);
        }
        reinterpret_cast<uint4*>(useg)[c - c0] = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
    __syncthreads();
    // output chunk c: group c / 4, pairs 4 (c % 4) .. + 3 = features
    // 4 (c % 4) .. + 3 (low halves) and 16 + 4 (c % 4) .. + 3 (high halves)
    for (int64_t c = tid; c < segn / 8; c += 256) {
      const int64_t grp = c >> 2, q4 = c & 3;
      const uint2 lo = reinterpret_cast<const uint2*>(useg)[grp * 8 + q4];      // features 4 q4 ..
      const uint2 hi = reinterpret_cast<const uint2*>(useg)[grp * 8 + 4 + q4];  // 16 + 4 q4 ..
      uint4 w;
      w.x = (lo.x & 0xFFFFu) | (hi.x << 16);
      w.y = (lo.x >> 16) | (hi.x & 0xFFFF0000u);
      w.z = (lo.y & 0xFFFFu) | (hi.y << 16);
      w.w = (lo.y >> 16) | (hi.y & 0xFFFF0000u);
      reinterpret_cast<uint4*>(out + seg)[c] = w;
    }
    __syncthreads();
  }
  // sum_m |u| at the true scale (sigma is a power of two: exact)
  acc = block_reduce(acc, true, red);
  if (tid == 0) p.l1[row] = acc / sig;
}

// ---- the two products -------------------------------------------------
struct GemmArgs {
  int stage;  // 1 or 2
  int L;
  int64_t T, K, kp, ncols;  // per-term contraction length (and padded), columns
  int64_t nkb, nrt;         // bit layout of the sign matrix (rows = ncols)
  int kw;
  int ntt, ntc;             // token tiles, column tiles of this launch
  const uint32_t* bits[DBF_MAX_TERMS];
  const uint16_t* colscale[DBF_MAX_TERMS];  // beta (stage 1) / alpha (stage 2)
  const _Float16* a;        // A operand [L][T][kp] in pair order
  const float* l1;          // [L][T]
  const float* bmax;        // [L]
  const float* sig;         // [T] prep's per-token power of two
  int sig_div;              // stage 2 reads u itself (boolean kernels): divide by sig too
  int nsplit;               // K-splits (grid z); > 1: fp32 partials to `part`
  float* part;              // [nsplit][terms in grid][T][ldp]
  int64_t ldp;
  _Float16* v;              // stage-1 output [L][T][vp] in pair order
  int64_t vp;
  void* y;
  int y_dtype;
  int64_t ldy;
  int accumulate;
};

// B fragment (8 fp16) for word `wd` (sign-folded: a set bit is a negative
// value) and feature pairs j = 8 * sub + 4 * h + q (q < 4) with j + 16:
// per pair one shift puts bits j and j + 16 on the two fp16 sign bits and
// one v_bfi_b32 merges in the magnitude pair `mag`.  `mag` must come from
// opaque() so that the compiler cannot see its clear sign bits and turn the
// bit insert back into an AND and an OR.
__device__ __forceinline__ half8 unpack_frag(uint32_t wd, int h, int sub, uint32_t mag) {
  const uint32_t v = wd >> (4 * h);
  uint32_t o[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    o[q] = ((v << (15 - 8 * sub - q)) & 0x80008000u) | (mag & 0x7FFF7FFFu);
  return __builtin_bit_cast(half8, make_uint4(o[0], o[1], o[2], o[3]));
}

// The value unchanged, but unknown to the optimizer (emits no instruction).
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm("" : "+v"(v));
  return v;
}

// Wait for this wave's vector-memory operations down to n outstanding, then
// a workgroup barrier; the signal fences keep the compiler from moving
// memory operations across either.
template <int N>
__device__ __forceinline__ void wait_then_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(N));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// STAGE 1: one term per grid row (blockIdx.y); STAGE 2: all terms in turn.
// KW4: the sign matrix has 4 words per row per tile (K >= 97); otherwise a
// single K-block of kw words per row.
// NB: LDS stages.  Each K step's operands (the BM x 128 fp16 A tile and, with
// KW4, the 16 bytes of sign words of each of the BN columns) are copied
// global -> LDS directly (global_load_lds_dwordx4, no register staging),
// NB - 1 steps ahead of the MFMAs.  A rows are stored unpadded, 16-byte chunk
// c of row r at chunk c ^ (r & 15), so the ds_read_b128 fragment reads of 16
// consecutive rows hit 16 different chunk slots (all 64 banks, no conflict).
template <int STAGE, bool KW4, int BM, int BN, int NB>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
gemm_kernel(GemmArgs p) {
  constexpr int RB = BM / 32;            // 32-token row blocks per wave
  constexpr int CB = BN / 128;           // 32-column blocks per wave
  constexpr int ACH = BM * (BK / 8) / kThreads;  // A chunks (16 B) per thread per step
  constexpr int LPS = ACH + (KW4 ? 1 : 0);       // loads per thread per step
  constexpr int ABYTES = BM * BK * 2;
  constexpr int SBYTES = ABYTES + (KW4 ? BN * 16 : 0);
  static_assert(LPS * (NB - 2) < 64, "vmcnt range");
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __shared__ float tokscale[BM];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int li = lane & 31, h = lane >> 5;

  const int ntiles = p.ntt * p.ntc;
  int b = blockIdx.x;
  if (ntiles % 8 == 0) b = (b & 7) * (ntiles >> 3) + (b >> 3);
  const int ttile = b / p.ntc, ctile = b - ttile * p.ntc;
  const int64_t tok0 = static_cast<int64_t>(ttile) * BM;
  const int64_t col0 = static_cast<int64_t>(ctile) * BN;
  const int term_first = STAGE == 1 ? static_cast<int>(blockIdx.y) : 0;
  const int term_end = STAGE == 1 ? term_first + 1 : p.L;

  // Inputs of the epilogue's per-token scale (stage 1: the factor s_t /
  // sigma_t of v; stage 2: the divisor s_t of y, s_t sigma_t when the A
  // operand is u itself).  Every thread loads them here (token clamped, term
  // slots past L repeating the last) and they are used only after the K
  // loop, so no wait for them stands before the first copies.  A K split
  // writes raw partial sums and does not use them.
  float tl1[DBF_MAX_TERMS], tbm[DBF_MAX_TERMS], tsig = 1.f;
  if (p.nsplit == 1) {
    const int64_t ttok = min<int64_t>(tok0 + tid % BM, p.T - 1);
#pragma unroll
    for (int i = 0; i < DBF_MAX_TERMS; ++i) {
      const int ii = min(i, p.L - 1);
      tbm[i] = p.bmax[ii];
      tl1[i] = p.l1[static_cast<int64_t>(ii) * p.T + ttok];
    }
    tsig = p.sig[ttok];
  }

  const int spt = static_cast<int>(p.kp / BK);  // K steps per term
  // this workgroup's K-split: steps [lo, hi) of the (term, step) sequence
  const int split = static_cast<int>(blockIdx.z);
  const int total = (term_end - term_first) * spt;
  const int lo = static_cast<int>(static_cast<int64_t>(total) * split / p.nsplit);
  const int hi = static_cast<int>(static_cast<int64_t>(total) * (split + 1) / p.nsplit);

  // this thread's A chunks: LDS chunk q * 256 + tid of a stage is row
  // (q * 256 + tid) / 16, slot tid % 16, and holds logical chunk
  // slot ^ (row & 15).  Rows past T read row T - 1 (never stored).
  int64_t aoff[ACH];
#pragma unroll
  for (int q = 0; q < ACH; ++q) {
    const int row = (q * kThreads + tid) >> 4;
    const int c = (tid & 15) ^ (row & 15);
    const int64_t tok = min(tok0 + row, p.T - 1);
    aoff[q] = tok * p.kp + 8 * c;
  }
  // sign words: column col0 + j (j < BN) of a stage at byte ABYTES + 16 j;
  // wave wv copies columns [wv * BN / 4, (wv + 1) * BN / 4)
  int64_t boff = 0;
  bool blane = true;
  if constexpr (KW4) {
    blane = lane < BN / 4;
    const int64_t col = col0 + (BN / 4) * wv + lane;
    const int64_t c = col < p.nrt * 64 ? col : 0;
    boff = ((c >> 6) * p.nkb * 64 + (c & 63)) * 4;
  }
  // this lane's MFMA columns
  int64_t bcol[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) bcol[cb] = col0 + (BN / 4) * wv + 32 * cb + li;

  // load cursor: (term, step within the term), advanced one step at a time
  int lterm = term_first + lo / spt, lks = lo % spt;
  // LDS byte address of the stages (the low 32 bits of the shared-aperture
  // address are the LDS offset)
  const unsigned lds0 = static_cast<unsigned>(reinterpret_cast<uintptr_t>(smem_raw));
  auto issue = [&](int stage_slot) {
    const unsigned st = lds0 + stage_slot * SBYTES;
    const _Float16* base = p.a + static_cast<int64_t>(lterm) * p.T * p.kp + lks * BK;
#pragma unroll
    for (int q = 0; q < ACH; ++q) copy16_to_lds(base + aoff[q], st + q * 4096 + wv * 1024);
    if constexpr (KW4) {
      if (blane)
        copy16_to_lds(p.bits[lterm] + boff + static_cast<int64_t>(lks) * 256,
                      st + ABYTES + wv * (BN / 4) * 16);
    }
    if (++lks == spt) {
      lks = 0;
      ++lterm;
    }
  };

  // sign fold and magnitude per column block (stage 2: +-|alpha|, stage 1: +-1)
  uint32_t flip[CB], mag[CB];
  // With one term, stage 2 applies alpha in the epilogue instead, so its
  // sign operand is +-1 as in stage 1 (fewer toggling operand bits: the
  // matrix cores run measurably faster on them).
  const bool fold_alpha = STAGE == 2 && p.L > 1;
  // Column scales with the column clamped (zero past ncols is applied where
  // they are used), loaded ahead of their use: the epilogue's (beta in
  // stage 1, alpha of a single term in stage 2) before the K loop, and with
  // several terms the next term's alpha for the sign fold when a term
  // starts, so that a term change inside the loop does not wait for memory.
  int64_t ccol[CB];
  uint16_t cscale[CB], anext[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    ccol[cb] = min<int64_t>(bcol[cb], p.ncols - 1);
    cscale[cb] = p.colscale[STAGE == 1 ? term_first : 0][ccol[cb]];
  }
  auto load_alpha = [&](int term) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) anext[cb] = p.colscale[min(term, p.L - 1)][ccol[cb]];
  };
  auto set_term = [&](int term) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      if (!fold_alpha) {
        flip[cb] = 0xFFFFFFFFu;           // bit 1 (+1) -> sign bit 0
        mag[cb] = opaque(0x3C003C00u);    // 1.0, 1.0
      } else {
        const uint16_t a = bcol[cb] < p.ncols ? anext[cb] : uint16_t(0);
        flip[cb] = (a & 0x8000u) ? 0u : 0xFFFFFFFFu;
        const uint32_t m = a & 0x7FFFu;
        mag[cb] = opaque(m | (m << 16));
      }
    }
  };

  floatx16 acc[RB][CB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rb][cb][r] = 0.f;

  const int nsteps = hi - lo;
#pragma unroll
  for (int j = 0; j < NB - 1; ++j)
    if (j < nsteps) issue(j);
  int cterm = term_first + lo / spt, cks = lo % spt;  // compute cursor
  if (fold_alpha) load_alpha(cterm);
  set_term(cterm);
  if (fold_alpha) load_alpha(cterm + 1);
  for (int step = 0; step < nsteps; ++step) {
    // this step's copies are done once at most (later steps issued) * LPS
    // of this wave's loads are still in flight; then all waves' are
    const int later = min(NB - 2, nsteps - 1 - step);
    if constexpr (NB == 2) {
      wait_then_barrier<0>();
    } else {
      if (later >= NB - 2) wait_then_barrier<LPS * (NB - 2)>();
      else if (NB >= 4 && later == 1) wait_then_barrier<LPS>();
      else wait_then_barrier<0>();
    }
    // the stage read one step ago is free again
    if (step + NB - 1 < nsteps) issue((step + NB - 1) % NB);
    const unsigned char* st = smem_raw + (step % NB) * SBYTES;
    uint32_t cw[CB][4];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      if constexpr (KW4) {
        const uint4 w4 = *reinterpret_cast<const uint4*>(st + ABYTES + ((BN / 4) * wv + 32 * cb + li) * 16);
        cw[cb][0] = w4.x; cw[cb][1] = w4.y; cw[cb][2] = w4.z; cw[cb][3] = w4.w;
      } else {
        // a single K-block of kw < 4 words per row (one step per term)
        const int64_t col = bcol[cb];
        const uint32_t* src = p.bits[cterm] + ((col >> 6) * 64 + (col & 63)) * p.kw;
#pragma unroll
        for (int j = 0; j < 4; ++j) cw[cb][j] = (j < p.kw && col < p.nrt * 64) ? src[j] : 0u;
      }
    }
    // 8 sub-steps of 16 features (wi, sub); the A fragments and sign values
    // of sub-step kk + 1 are fetched before the MFMAs of kk (the compiler
    // schedules them)
    half8 af[2][RB], bf[2][CB];
    auto fetch = [&](int kk, int slot) {
      const int wi = kk >> 1, sub = kk & 1;
      const int c = 4 * wi + 2 * sub + h;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int row = 32 * rb + li;
        af[slot][rb] = *reinterpret_cast<const half8*>(st + row * (BK * 2) + ((c ^ (row & 15)) << 4));
      }
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        bf[slot][cb] = unpack_frag(cw[cb][wi] ^ flip[cb], h, sub, mag[cb]);
    };
    fetch(0, 0);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      if (kk + 1 < 8) fetch(kk + 1, (kk + 1) & 1);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[kk & 1][rb], bf[kk & 1][cb],
                                                               acc[rb][cb], 0, 0, 0);
    }
    if (STAGE == 2 && ++cks == spt) {
      cks = 0;
      if (++cterm < term_end) {
        set_term(cterm);
        if (fold_alpha) load_alpha(cterm + 1);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  // epilogue; D layout: lane l, register r -> column l % 32,
  // row 8 * (r / 4) + 4 * (l / 32) + r % 4 of the 32 x 32 block.  Each wave
  // stages one 32-column block at a time in its own LDS slice (the stage
  // buffers are free now) and writes it out as 16-byte row chunks.
  const bool partial = p.nsplit > 1;
  if (!partial && tid < BM) {
    float bnd = 0.f;
#pragma unroll
    for (int i = 0; i < DBF_MAX_TERMS; ++i) bnd = fmaxf(bnd, tbm[i] * tl1[i]);
    float ts = 1.f;
    if (tok0 + tid < p.T) {
      ts = scale_from_bound(bnd);
      if (STAGE == 1) ts /= tsig;
      else if (p.sig_div) ts *= tsig;
    }
    tokscale[tid] = ts;
  }
  __syncthreads();  // every wave is done with the stage buffers; tokscale written
  unsigned char* wbuf = smem_raw + wv * (BM * 32 * 4);
  // staged element: fp16 v; y as stored, or fp32 when adding to y (one
  // rounding of old + new); fp32 partial sums when K is split
  const int esize = partial ? 4 : (STAGE == 1 ? 2 : ((p.y_dtype == DBF_F32 || p.accumulate) ? 4 : 2));
  const int cpr = 32 * esize / 16;  // 16-byte chunks per staged row
  const bool vec_y = STAGE == 2 && !p.accumulate && (p.ldy * esize) % 16 == 0;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int64_t c0 = col0 + (BN / 4) * wv + 32 * cb;  // first column of the block
    if (partial) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rl = 32 * rb + 8 * (r >> 2) + 4 * h + (r & 3);
          reinterpret_cast<float*>(wbuf)[rl * 32 + li] = acc[rb][cb][r];
        }
    } else if constexpr (STAGE == 1) {
      // v = fp16(s_t * beta_r * acc) at the pair-order position of r
      const float bsc = bcol[cb] < p.ncols ? f16_bits_to_f32(cscale[cb]) : 0.f;
      const int pos = li < 16 ? 2 * li : 2 * (li - 16) + 1;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rl = 32 * rb + 8 * (r >> 2) + 4 * h + (r & 3);
          reinterpret_cast<_Float16*>(wbuf)[rl * 32 + pos] =
              static_cast<_Float16>(tokscale[rl] * bsc * acc[rb][cb][r]);
        }
    } else {
      const float asc = (!fold_alpha && bcol[cb] < p.ncols) ? f16_bits_to_f32(cscale[cb]) : 1.f;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rl = 32 * rb + 8 * (r >> 2) + 4 * h + (r & 3);
          const float o = asc * acc[rb][cb][r] / tokscale[rl];
          if (esize == 4)
            reinterpret_cast<float*>(wbuf)[rl * 32 + li] = o;
          else
            reinterpret_cast<uint16_t*>(wbuf)[rl * 32 + li] =
                p.y_dtype == DBF_BF16 ? f32_to_bf16_bits(o) : f32_to_f16_bits(o);
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");  // slice written by the whole wave
    for (int c = lane; c < BM * cpr; c += 64) {
      const int row = c / cpr, ch = c - row * cpr;
      const int64_t tok = tok0 + row;
      if (tok >= p.T) continue;
      const uint4 d = reinterpret_cast<const uint4*>(wbuf)[c];
      if (partial) {
        // 4 columns; columns past ncols (up to ldp) are never read
        const int64_t col = c0 + 4 * ch;
        const int64_t prow = (static_cast<int64_t>(split) * gridDim.y + blockIdx.y) * p.T + tok;
        if (col < p.ldp) *reinterpret_cast<uint4*>(p.part + prow * p.ldp + col) = d;
      } else if constexpr (STAGE == 1) {
        // 8 positions of the 32-position group of this block
        const int64_t pos = c0 + 8 * ch;
        if (pos < p.vp)
          *reinterpret_cast<uint4*>(p.v + (static_cast<int64_t>(term_first) * p.T + tok) * p.vp + pos) = d;
      } else {
        const int per = 16 / esize;
        const int64_t col = c0 + per * ch;
        if (vec_y && col + per <= p.ncols) {
          *reinterpret_cast<uint4*>(static_cast<unsigned char*>(p.y) + (tok * p.ldy + col) * esize) = d;
        } else {
          const uint32_t w[4] = {d.x, d.y, d.z, d.w};
          for (int e = 0; e < per; ++e) {
            if (col + e >= p.ncols) break;
            float v;
            if (esize == 4)
              v = __uint_as_float(w[e]);
            else {
              const uint16_t b = static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1)));
              v = p.y_dtype == DBF_BF16 ? bf16_bits_to_f32(b) : f16_bits_to_f32(b);
            }
            store_out(p.y, p.y_dtype, tok * p.ldy + col + e, v, p.accumulate);
          }
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");  // slice read before reuse
  }
}

// ---- K-split reductions ------------------------------------------------
constexpr int kSplitTarget = 256;  // workgroups a split product aims for
constexpr int kMaxSplit = 16;
constexpr int64_t kShortSteps = 32;

// Stage 1: v_i[t, pos] = fp16(s_t * beta_i[r] * sum_split part[split][i][t][r])
// for the 8 pair-order positions of one 16-byte chunk (pairs j .. j + 3 of a
// 32-feature group: r = 32 g + j and 32 g + 16 + j); zero past R.  The
// splits are added in order, so the result does not depend on timing.
struct Reduce1Args {
  const float* part;
  int64_t ldp, T, R, vp;
  int L, nsplit;
  const uint16_t* beta[DBF_MAX_TERMS];
  const float* l1;
  const float* bmax;
  const float* sig;
  _Float16* v;
};

// NS = nsplit.  A thread's loads (scales, every split's partials, beta) are
// all issued before the first of them is used, with addresses clamped into
// the buffers instead of branches around the loads, so that the kernel
// waits for memory once.
// Grid: (ceil(T * vp / 8 / 256), L); the term is the grid row, so its beta
// pointer is a scalar load.
template <int NS>
__global__ void __launch_bounds__(256) reduce1_kernel(Reduce1Args p) {
  const int64_t nch = p.vp / 8;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= p.T * nch) return;
  const int term = static_cast<int>(blockIdx.y);
  const int64_t tok = idx / nch;
  const int64_t c = idx - tok * nch;
  const int64_t row = static_cast<int64_t>(term) * p.T + tok;
  const int64_t r0[2] = {32 * (c >> 2) + 4 * (c & 3), 32 * (c >> 2) + 16 + 4 * (c & 3)};
  const int64_t sstride = static_cast<int64_t>(p.L) * p.T * p.ldp;
  // a chunk that starts past R reads the row's last chunk (its outputs are
  // zero); one that starts below R lies inside the row (ldp = R rounded up to 4)
  float4 q[NS][2];
#pragma unroll
  for (int sp = 0; sp < NS; ++sp)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      q[sp][hh] = *reinterpret_cast<const float4*>(p.part + sp * sstride + row * p.ldp +
                                                   min(r0[hh], p.ldp - 4));
  const uint16_t* bt = p.beta[term];
  uint16_t bb[2][4];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int e = 0; e < 4; ++e) bb[hh][e] = bt[min(r0[hh] + e, p.R - 1)];
  const float sig = p.sig[tok];
  const float sc = scale_from_bound(term_bound(p.bmax, p.l1, p.L, p.T, tok)) / sig;
  // the sums in split order
  float sum[2][4] = {};
#pragma unroll
  for (int sp = 0; sp < NS; ++sp)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      sum[hh][0] += q[sp][hh].x; sum[hh][1] += q[sp][hh].y;
      sum[hh][2] += q[sp][hh].z; sum[hh][3] += q[sp][hh].w;
    }
  // positions past R are zeroed with a mask the optimizer cannot see through:
  // a select there would become a branch with the loads sunk into it
  uint32_t o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint32_t hb[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const _Float16 hv = static_cast<_Float16>(sc * f16_bits_to_f32(bb[hh][e]) * sum[hh][e]);
      hb[hh] = __builtin_bit_cast(uint16_t, hv) & opaque(r0[hh] + e < p.R ? 0xFFFFu : 0u);
    }
    o[e] = hb[0] | (hb[1] << 16);
  }
  *reinterpret_cast<uint4*>(p.v + row * p.vp + 8 * c) = make_uint4(o[0], o[1], o[2], o[3]);
}

// Stage 2: y[t, n] (+)= a_n / s_t * sum_split part[split][t][n], a_n = alpha_n
// with one term (alpha not folded into the signs), else 1; 4 columns a thread.
struct Reduce2Args {
  const float* part;
  int64_t ldp, T, N;
  int L, nsplit;
  const uint16_t* alpha;
  const float* l1;
  const float* bmax;
  const float* sig;
  int sig_div;
  void* y;
  int y_dtype;
  int64_t ldy;
  int accumulate;
};

// NS = nsplit; loads issued as in reduce1_kernel.  Four whole columns are
// written with one store when y's layout allows it.
template <int NS>
__global__ void __launch_bounds__(256) reduce2_kernel(Reduce2Args p) {
  const int64_t nch = (p.N + 3) / 4;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= p.T * nch) return;
  const int64_t tok = idx / nch;
  const int64_t n0 = 4 * (idx - tok * nch);  // n0 + 4 <= ldp (N rounded up to 4)
  float4 q[NS];
#pragma unroll
  for (int sp = 0; sp < NS; ++sp)
    q[sp] = *reinterpret_cast<const float4*>(p.part + (sp * p.T + tok) * p.ldp + n0);
  uint16_t ab[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) ab[e] = p.alpha[min(n0 + e, p.N - 1)];
  const float sg = p.sig[tok];
  const float sc = scale_from_bound(term_bound(p.bmax, p.l1, p.L, p.T, tok)) * (p.sig_div ? sg : 1.f);
  float sum[4] = {};
#pragma unroll
  for (int sp = 0; sp < NS; ++sp) {
    sum[0] += q[sp].x; sum[1] += q[sp].y; sum[2] += q[sp].z; sum[3] += q[sp].w;
  }
  // alpha with one term, else 1, chosen by a mask (a select would become a
  // branch with the alpha loads sunk into it)
  const uint32_t one_term = opaque(p.L == 1 ? 0xFFFFu : 0u);
  float o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    o[e] = f16_bits_to_f32(static_cast<uint16_t>((ab[e] & one_term) | (0x3C00u & ~one_term))) * sum[e] / sc;
  const int64_t at = tok * p.ldy + n0;
  if (!p.accumulate && n0 + 4 <= p.N) {
    if (p.y_dtype == DBF_F32) {
      float* dst = static_cast<float*>(p.y) + at;
      if (reinterpret_cast<uintptr_t>(dst) % 16 == 0) {
        *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
        return;
      }
    } else {
      uint16_t* dst = static_cast<uint16_t*>(p.y) + at;
      if (reinterpret_cast<uintptr_t>(dst) % 8 == 0) {
        uint32_t w[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t lo = p.y_dtype == DBF_BF16 ? f32_to_bf16_bits(o[2 * h]) : f32_to_f16_bits(o[2 * h]);
          const uint32_t hi = p.y_dtype == DBF_BF16 ? f32_to_bf16_bits(o[2 * h + 1])
                                                    : f32_to_f16_bits(o[2 * h + 1]);
          w[h] = lo | (hi << 16);
        }
        *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
        return;
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (n0 + e >= p.N) break;
    store_out(p.y, p.y_dtype, at + e, o[e], p.accumulate);
  }
}

// Launch the reduction instantiated for the split count (2 .. kMaxSplit).
template <int NS = 2>
hipError_t launch_reduce1(const Reduce1Args& r, dim3 grid, hipStream_t s) {
  if constexpr (NS > kMaxSplit) {
    return hipErrorInvalidValue;
  } else {
    if (r.nsplit != NS) return launch_reduce1<NS + 1>(r, grid, s);
    reduce1_kernel<NS><<<grid, 256, 0, s>>>(r);
    return hipGetLastError();
  }
}

template <int NS = 2>
hipError_t launch_reduce2(const Reduce2Args& r, dim3 grid, hipStream_t s) {
  if constexpr (NS > kMaxSplit) {
    return hipErrorInvalidValue;
  } else {
    if (r.nsplit != NS) return launch_reduce2<NS + 1>(r, grid, s);
    reduce2_kernel<NS><<<grid, 256, 0, s>>>(r);
    return hipGetLastError();
  }
}

// Tile shape and K-split of one product: the largest of 128 x 256,
// 128 x 128, 64 x 128 that still gives >= 256 workgroups, where a short
// product (at most kShortSteps K steps), or one of at most 32 tokens (one
// token tile either way, less padding), takes 32 x 128 tiles instead of
// 64 x 128 ones; with fewer tiles than that, K is split (each split >= 2
// steps, at most kMaxSplit) towards kSplitTarget workgroups, taking among
// up to twice the fewest such splits the count whose workgroups fill their
// last round of 256 best.  (Measured on MI355X for 16 to 256 tokens: a
// target of 256 beat 512 and 1024, the split partials' traffic growing with
// the split count; but 86 tiles split 3 ways are 258 workgroups, two past a
// round, and 5 ways (430) ran 11008 x 4096 products 4-20% faster, three
// boolean kernels at 8 tokens 40.2 -> 32.3 us.  32-row tiles, which halve
// the split, beat 64-row ones on products of 16 and 32 steps: 4096 x 4096
// R 2048 at 64 tokens 33.2 -> 28.4 us, at 256 tokens 42.3 -> 37.7 us; on
// products of 48 and 64 steps they lost, 51.6 -> 53.5 us and 40.7 -> 46.0
// us, each sign unpack serving one MFMA instead of two.)

struct Tiling {
  int bm, bn, ntt, ntc, nsplit;
};

Tiling choose_tiling(int64_t T, int64_t cols, int terms_in_grid, int64_t steps) {
  auto wgs = [&](int bm, int bn) { return cdiv(T, bm) * cdiv(cols, bn) * terms_in_grid; };
  Tiling t{128, 256, 0, 0, 1};
  if (wgs(128, 256) < 256) t.bn = 128;
  if (wgs(128, 128) < 256) t.bm = 64;
  if (wgs(64, 128) < 256 && (steps <= kShortSteps || T <= 32)) t.bm = 32;
  t.ntt = static_cast<int>(cdiv(T, t.bm));
  t.ntc = static_cast<int>(cdiv(cols, t.bn));
  const int64_t tiles = wgs(t.bm, t.bn);
  if (tiles < 256) {
    // from the fewest splits that reach kSplitTarget workgroups up to twice
    // as many, the count whose last round of 256 workgroups is fullest
    const int64_t cap = std::max<int64_t>(1, std::min<int64_t>(steps / 2, kMaxSplit));
    const int64_t sp0 = std::min<int64_t>(cdiv(kSplitTarget, tiles), cap);
    int64_t best = sp0;
    double best_fill = 0.0;
    for (int64_t sp = sp0; sp <= std::min<int64_t>(2 * sp0, cap); ++sp) {
      const int64_t n = tiles * sp;
      const double fill = static_cast<double>(n) / (256.0 * static_cast<double>(cdiv(n, 256)));
      if (fill > best_fill + 1e-9) {
        best_fill = fill;
        best = sp;
      }
    }
    t.nsplit = static_cast<int>(std::max<int64_t>(best, 1));
  }
  return t;
}


template <int STAGE, bool KW4>
hipError_t launch_tiled(GemmArgs& a, const Tiling& tl, int terms_in_grid, hipStream_t s) {
  a.ntt = tl.ntt;
  a.ntc = tl.ntc;
  a.nsplit = tl.nsplit;
  const dim3 grid(static_cast<unsigned>(a.ntt * a.ntc), terms_in_grid, tl.nsplit);
  auto go = [&](auto kern, size_t lds) -> hipError_t {
    static bool attr_set = false;  // per instantiation; idempotent if raced
    if (!attr_set) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               static_cast<int>(lds));
      if (e != hipSuccess) return e;
      attr_set = true;
    }
    kern<<<grid, kThreads, lds, s>>>(a);
    return hipGetLastError();
  };
  // LDS per stage: the fp16 A tile plus (KW4) 16 bytes of sign words per column
  auto lds_of = [](int bm_, int bn_, int nb_) {
    return static_cast<size_t>(nb_) * (static_cast<size_t>(bm_) * BK * 2 + (KW4 ? bn_ * 16 : 0));
  };
  if (tl.bm == 128 && tl.bn == 256) return go(gemm_kernel<STAGE, KW4, 128, 256, kStages>, lds_of(128, 256, kStages));
  if (tl.bm == 128) return go(gemm_kernel<STAGE, KW4, 128, 128, kStages>, lds_of(128, 128, kStages));
  if (tl.bm == 32) return go(gemm_kernel<STAGE, KW4, 32, 128, kStages>, lds_of(32, 128, kStages));
  return go(gemm_kernel<STAGE, KW4, 64, 128, kStages>, lds_of(64, 128, kStages));
}

template <int STAGE>
hipError_t launch_stage(GemmArgs& a, const Tiling& tl, int terms_in_grid, hipStream_t s) {
  return a.kw == 4 ? launch_tiled<STAGE, true>(a, tl, terms_in_grid, s)
                   : launch_tiled<STAGE, false>(a, tl, terms_in_grid, s);
}

int64_t round4(int64_t n) { return (n + 3) / 4 * 4; }

// The two products' tilings (stage 1: R columns, one term per grid row,
// kpad(M) / BK steps; stage 2: N columns, all terms, L kpad(R) / BK steps).
struct Plan {
  Tiling t1, t2;
};

Plan make_plan(int64_t N, int64_t M, int64_t R, int L, int64_t T) {
  Plan pl;
  pl.t1 = choose_tiling(T, R, L, kpad(M) / BK);
  pl.t2 = choose_tiling(T, N, 1, L * (kpad(R) / BK));
  return pl;
}

// prep: L max|beta| workgroups, then one per (term, token)
hipError_t launch_prep(const PrepArgs& pa, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(pa.L * pa.T + pa.L));
  const bool x32 = pa.vec == 2;
  if (pa.L == 1) {
    if (x32) prep_kernel<0, true><<<grid, 256, 0, s>>>(pa);
    else prep_kernel<0, false><<<grid, 256, 0, s>>>(pa);
  } else if (pa.L == 2) {
    if (x32) prep_kernel<2, true><<<grid, 256, 0, s>>>(pa);
    else prep_kernel<2, false><<<grid, 256, 0, s>>>(pa);
  } else {
    if (x32) prep_kernel<4, true><<<grid, 256, 0, s>>>(pa);
    else prep_kernel<4, false><<<grid, 256, 0, s>>>(pa);
  }
  return hipGetLastError();
}

struct WsLayout {
  size_t u, v, l1, bmax, sig, part, total;
};

WsLayout ws_layout(int64_t N, int64_t M, int64_t R, int L, int64_t T) {
  auto al = [](size_t n) { return (n + 255) / 256 * 256; };
  const Plan pl = make_plan(N, M, R, L, T);
  WsLayout w{};
  size_t off = kWsHeadBytes;
  w.u = off; off += al(static_cast<size_t>(L) * T * kpad(M) * 2);
  w.v = off; off += al(static_cast<size_t>(L) * T * kpad(R) * 2);
  w.l1 = off; off += al(static_cast<size_t>(L) * T * 4);
  w.bmax = off; off += al(static_cast<size_t>(L) * 4);
  w.sig = off; off += al(static_cast<size_t>(T) * 4);
  // split partials: stage 1's are consumed before stage 2 writes its own
  size_t part = 0;
  if (pl.t1.nsplit > 1) part = static_cast<size_t>(pl.t1.nsplit) * L * T * round4(R) * 4;
  if (pl.t2.nsplit > 1) part = std::max(part, static_cast<size_t>(pl.t2.nsplit) * T * round4(N) * 4);
  w.part = off; off += al(part);
  w.total = off;
  return w;
}

}  // namespace

size_t mfma_ws_bytes(int64_t N, int64_t M, int64_t R, int n_terms, int64_t T) {
  return ws_layout(N, M, R, n_terms, T).total;
}

namespace {

// Boolean kernels: u_k [L][T][kpad(M)], per-token sums, max|s| slots (zero),
// then the split partials of the one product.
struct BoolLayout {
  size_t u, l1, bmax, sig, part, total;
  Tiling tl;
};

BoolLayout bool_layout(int64_t N, int64_t M, int L, int64_t T) {
  auto al = [](size_t n) { return (n + 255) / 256 * 256; };
  BoolLayout w{};
  w.tl = choose_tiling(T, N, 1, L * (kpad(M) / BK));
  size_t off = kWsHeadBytes;
  w.u = off; off += al(static_cast<size_t>(L) * T * kpad(M) * 2);
  w.l1 = off; off += al(static_cast<size_t>(L) * T * 4);
  w.bmax = off; off += al(static_cast<size_t>(L) * 4);
  w.sig = off; off += al(static_cast<size_t>(T) * 4);
  w.part = off;
  if (w.tl.nsplit > 1) off += al(static_cast<size_t>(w.tl.nsplit) * T * round4(N) * 4);
  w.total = off;
  return w;
}

}  // namespace

size_t mfma_bool_ws_bytes(int64_t N, int64_t M, int n_kernels, int64_t T) {
  return bool_layout(N, M, n_kernels, T).total;
}

// y = sum_k s_out_k . (Wb_k u_k) / sigma_t, u_k = fp16(sigma_t s_in_k . x):
// prep, then the stage-2 product with the sign matrices in the place of B1
// and u in the place of v.  prep sees no beta (R = 0), so max|beta| is 0 and
// s_t is exactly 1: the product divides by sigma_t alone.
hipError_t launch_bool_mfma(const TermPtrs& t, int64_t N, int64_t M, const void* x,
                            int x_dtype, int64_t T, int64_t ldx, void* y, int y_dtype,
                            int64_t ldy, int accumulate, void* ws, hipStream_t s) {
  unsigned char* base = static_cast<unsigned char*>(ws);
  const BoolLayout lay = bool_layout(N, M, t.n, T);
  _Float16* u = reinterpret_cast<_Float16*>(base + lay.u);
  float* l1 = reinterpret_cast<float*>(base + lay.l1);
  float* bmax = reinterpret_cast<float*>(base + lay.bmax);
  float* sig = reinterpret_cast<float*>(base + lay.sig);
  float* part = reinterpret_cast<float*>(base + lay.part);

  PrepArgs pa{};
  pa.x = x; pa.x_dtype = x_dtype; pa.ldx = ldx; pa.T = T; pa.M = M; pa.mpad = kpad(M);
  pa.R = 0; pa.L = t.n; pa.u = u; pa.l1 = l1; pa.bmax = bmax; pa.sig = sig;
  // eight 16-bit activations per 16-byte load, or eight fp32 ones per two
  pa.vec = reinterpret_cast<uintptr_t>(x) % 16 != 0 ? 0
           : x_dtype == DBF_F32                    ? (ldx % 4 == 0 ? 2 : 0)
                                                   : (ldx % 8 == 0 ? 1 : 0);
  for (int i = 0; i < t.n; ++i) {
    if (reinterpret_cast<uintptr_t>(t.gamma[i]) % 16 != 0) pa.vec = 0;
    pa.gamma[i] = t.gamma[i];
    pa.beta[i] = nullptr;
  }
  hipError_t e = launch_prep(pa, s);
  if (e != hipSuccess) return e;

  GemmArgs b{};
  b.stage = 2; b.L = t.n; b.T = T; b.K = M; b.kp = kpad(M); b.ncols = N;
  b.nkb = layout_nkb(M); b.nrt = layout_nrt(N); b.kw = static_cast<int>(layout_kw(M));
  for (int i = 0; i < t.n; ++i) {
    b.bits[i] = t.b1[i];
    b.colscale[i] = t.alpha[i];
  }
  b.a = u; b.l1 = l1; b.bmax = bmax; b.sig = sig; b.sig_div = 1;
  b.y = y; b.y_dtype = y_dtype; b.ldy = ldy; b.accumulate = accumulate;
  b.part = part; b.ldp = round4(N);
  e = launch_stage<2>(b, lay.tl, 1, s);
  if (e != hipSuccess || lay.tl.nsplit == 1) return e;
  Reduce2Args r{};
  r.part = part; r.ldp = b.ldp; r.T = T; r.N = N; r.L = t.n; r.nsplit = lay.tl.nsplit;
  r.alpha = t.alpha[0]; r.l1 = l1; r.bmax = bmax; r.sig = sig; r.sig_div = 1;
  r.y = y; r.y_dtype = y_dtype; r.ldy = ldy; r.accumulate = accumulate;
  return launch_reduce2(r, dim3(static_cast<unsigned>(cdiv(T * cdiv(N, 4), 256))), s);
}

hipError_t launch_mfma(const TermPtrs& t, int64_t N, int64_t M, int64_t R,
                       const void* x, int x_dtype, int64_t T, int64_t ldx,
                       void* y, int y_dtype, int64_t ldy, int accumulate,
                       void* ws, hipStream_t s) {
  unsigned char* base = static_cast<unsigned char*>(ws);
  const WsLayout lay = ws_layout(N, M, R, t.n, T);
  const Plan pl = make_plan(N, M, R, t.n, T);
  float* part = reinterpret_cast<float*>(base + lay.part);
  _Float16* u = reinterpret_cast<_Float16*>(base + lay.u);
  _Float16* v = reinterpret_cast<_Float16*>(base + lay.v);
  float* l1 = reinterpret_cast<float*>(base + lay.l1);
  float* bmax = reinterpret_cast<float*>(base + lay.bmax);
  float* sig = reinterpret_cast<float*>(base + lay.sig);

  PrepArgs pa{};
  pa.x = x; pa.x_dtype = x_dtype; pa.ldx = ldx; pa.T = T; pa.M = M; pa.mpad = kpad(M);
  pa.R = R; pa.L = t.n; pa.u = u; pa.l1 = l1; pa.bmax = bmax; pa.sig = sig;
  pa.vec = (ldx % 8 == 0) && (reinterpret_cast<uintptr_t>(x) % 16 == 0);
  for (int i = 0; i < t.n; ++i)
    if (reinterpret_cast<uintptr_t>(t.gamma[i]) % 16 != 0) pa.vec = 0;
  for (int i = 0; i < t.n; ++i) {
    pa.gamma[i] = t.gamma[i];
    pa.beta[i] = t.beta[i];
  }
  hipError_t e = launch_prep(pa, s);
  if (e != hipSuccess) return e;

  GemmArgs a{};
  a.stage = 1; a.L = t.n; a.T = T; a.K = M; a.kp = kpad(M); a.ncols = R;
  a.nkb = layout_nkb(M); a.nrt = layout_nrt(R); a.kw = static_cast<int>(layout_kw(M));
  for (int i = 0; i < t.n; ++i) {
    a.bits[i] = t.b2[i];
    a.colscale[i] = t.beta[i];
  }
  a.a = u; a.l1 = l1; a.bmax = bmax; a.sig = sig; a.sig_div = 0; a.v = v; a.vp = kpad(R);
  a.part = part; a.ldp = round4(R);
  e = launch_stage<1>(a, pl.t1, t.n, s);
  if (e != hipSuccess) return e;
  if (pl.t1.nsplit > 1) {
    Reduce1Args r{};
    r.part = part; r.ldp = a.ldp; r.T = T; r.R = R; r.vp = a.vp; r.L = t.n;
    r.nsplit = pl.t1.nsplit; r.l1 = l1; r.bmax = bmax; r.sig = sig; r.v = v;
    for (int i = 0; i < t.n; ++i) r.beta[i] = t.beta[i];
    e = launch_reduce1(r, dim3(static_cast<unsigned>(cdiv(T * (a.vp / 8), 256)), t.n), s);
    if (e != hipSuccess) return e;
  }

  GemmArgs b = a;
  b.stage = 2; b.K = R; b.kp = kpad(R); b.ncols = N;
  b.nkb = layout_nkb(R); b.nrt = layout_nrt(N); b.kw = static_cast<int>(layout_kw(R));
  for (int i = 0; i < t.n; ++i) {
    b.bits[i] = t.b1[i];
    b.colscale[i] = t.alpha[i];
  }
  b.a = v;
  b.y = y; b.y_dtype = y_dtype; b.ldy = ldy; b.accumulate = accumulate;
  b.ldp = round4(N);
  e = launch_stage<2>(b, pl.t2, 1, s);
  if (e != hipSuccess || pl.t2.nsplit == 1) return e;
  Reduce2Args r{};
  r.part = part; r.ldp = b.ldp; r.T = T; r.N = N; r.L = t.n; r.nsplit = pl.t2.nsplit;
  r.alpha = t.alpha[0]; r.l1 = l1; r.bmax = bmax; r.sig = sig; r.sig_div = 0;
  r.y = y; r.y_dtype = y_dtype; r.ldy = ldy; r.accumulate = accumulate;
  return launch_reduce2(r, dim3(static_cast<unsigned>(cdiv(T * cdiv(N, 4), 256))), s);
}

}  // namespace dbf
