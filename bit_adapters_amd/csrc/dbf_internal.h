// Internal declarations shared by the HIP translation units of libdbf.
// Layout: see include/dbf.h (DBF_LAYOUT_VERSION 1).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>
#include <stddef.h>
#include <algorithm>

#include "dbf.h"

namespace dbf {

constexpr int kTileRows = 64;

// Words per row per tile, tiles along K, tiles along rows.
__host__ __device__ inline int64_t layout_kw(int64_t K) {
  int64_t w = (K + 31) / 32;
  return w < 1 ? 1 : (w > 4 ? 4 : w);
}
__host__ __device__ inline int64_t layout_nkb(int64_t K) {
  int64_t kw = layout_kw(K);
  return (K + 32 * kw - 1) / (32 * kw);
}
__host__ __device__ inline int64_t layout_nrt(int64_t rows) {
  return (rows + kTileRows - 1) / kTileRows;
}
__host__ __device__ inline int64_t layout_words(int64_t rows, int64_t K) {
  return layout_nrt(rows) * layout_nkb(K) * kTileRows * layout_kw(K);
}

// ---- scalar conversions (device) ------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return __half2float(__ushort_as_half(b));
}
// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  return __half_as_ushort(__float2half_rn(f));
}

// Power of two that brings the largest |v| of a set of values (a token's
// |scale_in . x|, say) into [2^14, 2^15), so that fp16(sigma . v) neither
// overflows nor leaves the normal range where it matters (a power of two
// commutes with the fp16 rounding wherever the result is normal).  1 for an
// all-zero (or non-finite) set.
__device__ __forceinline__ float act_scale(float amax) {
  if (!(amax > 0.f) || !(amax <= 3.0e38f)) return 1.f;
  int e = 0;
  frexpf(amax, &e);  // amax = f * 2^e, f in [0.5, 1)
  return ldexpf(1.f, max(-100, min(100, 15 - e)));
}

// Load element i of an activation array of dtype code dt (bf16, f16, or
// f32 for the backward's fp32 intermediates) as fp32.
__device__ __forceinline__ float load_act(const void* p, int dt, int64_t i) {
  if (dt == DBF_F32) return static_cast<const float*>(p)[i];
  const uint16_t v = static_cast<const uint16_t*>(p)[i];
  return dt == DBF_BF16 ? bf16_bits_to_f32(v) : f16_bits_to_f32(v);
}

// Store fp32 v into y (dtype dt) at i, optionally adding the old value.
__device__ __forceinline__ void store_out(void* y, int dt, int64_t i, float v,
                                          int accumulate) {
  if (dt == DBF_F32) {
    float* p = static_cast<float*>(y) + i;
    *p = accumulate ? *p + v : v;
  } else if (dt == DBF_BF16) {
    uint16_t* p = static_cast<uint16_t*>(y) + i;
    float o = accumulate ? bf16_bits_to_f32(*p) + v : v;
    *p = f32_to_bf16_bits(o);
  } else {
    uint16_t* p = static_cast<uint16_t*>(y) + i;
    float o = accumulate ? f16_bits_to_f32(*p) + v : v;
    *p = f32_to_f16_bits(o);
  }
}

// ---- global -> LDS copies -------------------------------------------------
// s_waitcnt immediate that waits until at most n vector-memory operations
// of this wave are outstanding (expcnt and lgkmcnt not waited on).
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }
// s_waitcnt immediate for this wave's LDS operations only (lgkmcnt(0)).
constexpr int lgkmcnt0_imm() { return 15 | (7 << 4) | (0 << 8) | (3 << 14); }

// Copy 16 (4) bytes per lane from global memory straight into LDS: lane l's
// bytes land at LDS byte address lds + 16 l (lds + 4 l); M0 = lds
// (global_load_lds_dwordx4 / global_load_lds_dword).  Written as inline asm
// so that the compiler does not guard every later LDS read with a wait for
// all such copies; the kernels wait for them themselves (s_waitcnt vmcnt)
// before reading the bytes.  The instructions have no register result, and
// their address registers are read when they issue.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is reserved; it is still clobbered
__device__ __forceinline__ void copy16_to_lds(const void* src, unsigned lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}
__device__ __forceinline__ void copy4_to_lds(const void* src, unsigned lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}
#pragma clang diagnostic pop

// ---- kernel launchers (host, internal C++) -------------------------------
// Each returns hipSuccess or the launch error; arguments are already
// validated by the ABI layer.

hipError_t launch_pack(const void* src, int src_dtype, int64_t rows, int64_t k,
                       int64_t ld, uint32_t* packed, hipStream_t s);
// out = the packed layout of S^T (k rows x `rows`) for the packed S.
hipError_t launch_transpose_packed(const uint32_t* packed, int64_t rows, int64_t k,
                                   uint32_t* out, hipStream_t s);
hipError_t launch_unpack(const uint32_t* packed, int64_t rows, int64_t k,
                         int8_t* dst, int64_t ld, hipStream_t s);

// Term arrays as passed to kernels (by value).
struct TermPtrs {
  const uint32_t* b1[DBF_MAX_TERMS];
  const uint32_t* b2[DBF_MAX_TERMS];
  const uint16_t* alpha[DBF_MAX_TERMS];
  const uint16_t* beta[DBF_MAX_TERMS];
  const uint16_t* gamma[DBF_MAX_TERMS];
  int n;
};

// Decode path (signed subset-sum tables).  ws: 256 bytes of counters, then
// fp32 partials of w = beta * (B2 u) as [n_terms][ks][T][R_pad].
size_t decode_ws_bytes(int64_t N, int64_t M, int64_t R, int n_terms, int64_t T);
hipError_t launch_decode(const TermPtrs& t, int64_t N, int64_t M, int64_t R,
                         const void* x, int x_dtype, int64_t T, int64_t ldx,
                         void* y, int y_dtype, int64_t ldy, int accumulate,
                         void* ws, hipStream_t s);
hipError_t launch_decode_i8(const TermPtrs& t, int64_t N, int64_t M, int64_t R,
                            const int8_t* x, int64_t T, int64_t ldx,
                            int32_t* s1, int32_t* s2, void* y, int y_dtype,
                            int64_t ldy, void* ws, hipStream_t s);

// Boolean kernels (Multi-Boolean form), decode path: t.b2 = the sign
// matrices [N x M], t.gamma = s_in, t.beta = s_out; workspace as
// decode_ws_bytes(N, M, N, n, T).
hipError_t launch_bool_decode(const TermPtrs& t, int64_t N, int64_t M, const void* x,
                              int x_dtype, int64_t T, int64_t ldx, void* y, int y_dtype,
                              int64_t ldy, int accumulate, void* ws, hipStream_t s);

// MFMA path.
size_t mfma_ws_bytes(int64_t N, int64_t M, int64_t R, int n_terms, int64_t T);
// Boolean kernels on the MFMA path: t.b1 = the sign matrices [N x M],
// t.gamma = s_in, t.alpha = s_out.
size_t mfma_bool_ws_bytes(int64_t N, int64_t M, int n_kernels, int64_t T);
hipError_t launch_bool_mfma(const TermPtrs& t, int64_t N, int64_t M, const void* x,
                            int x_dtype, int64_t T, int64_t ldx, void* y, int y_dtype,
                            int64_t ldy, int accumulate, void* ws, hipStream_t s);
hipError_t launch_mfma(const TermPtrs& t, int64_t N, int64_t M, int64_t R,
                       const void* x, int x_dtype, int64_t T, int64_t ldx,
                       void* y, int y_dtype, int64_t ldy, int accumulate,
                       void* ws, hipStream_t s);

// Backward (dx and the scale gradients) from four sign-accumulate products
// per term; b1t / b2t are the packed transposes of B1 / B2; path is
// DBF_PATH_DECODE or DBF_PATH_MFMA for every product.
size_t backward_ws_bytes(int64_t N, int64_t M, int64_t R, int n_terms, int64_t T, int path);
hipError_t launch_backward(const TermPtrs& t, const uint32_t* const* b1t,
                           const uint32_t* const* b2t, int64_t N, int64_t M, int64_t R,
                           const void* x, int x_dtype, int64_t ldx, const void* dy,
                           int dy_dtype, int64_t lddy, int64_t T, void* dx, int dx_dtype,
                           int64_t lddx, float* dalpha, float* dbeta, float* dgamma,
                           int path, void* ws, hipStream_t s);

// Successive SVID extraction (dbf_svid.hip): n_kernels boolean kernels of
// the real N x M matrix w (dtype w_dtype, row stride ldw) into the packed
// signs wb[k], fp16 s_in[k] [M] and s_out[k] [N]; residual_sq[k] (optional)
// = ||W - sum_{j <= k} kernel_j||_F^2; ws of svid_ws_bytes(N, M) bytes.
size_t svid_ws_bytes(int64_t N, int64_t M);
hipError_t launch_svid(const void* w, int w_dtype, int64_t N, int64_t M, int64_t ldw, int n_kernels,
                       uint32_t* const* wb, uint16_t* const* s_in, uint16_t* const* s_out, int iters,
                       float* residual_sq, void* ws, hipStream_t s);

// Several adapters, one per token (idx[t] in [-1, n_adapters), -1 = base
// only), in one launch: one-token stage-1 workgroups each run their
// token's adapter, the row workgroups stream the base once for every token
// and add each token's adapter term (adapters[a] has n = 1).
constexpr int kMaxAdapters = DBF_MAX_ADAPTERS;
hipError_t launch_multi_adapter(const uint16_t* w0, int64_t ldw, const TermPtrs* adapters,
                                int n_adapters, int64_t N, int64_t M, int64_t R,
                                const int32_t* idx, const void* x, int64_t T, int64_t ldx,
                                void* y, int y_dtype, int64_t ldy, void* ws, hipStream_t s);

// Adapter: y = W0 x + sum_i Delta W_i x in one launch (stage 1 of the
// decode path plus the base product; ws as for the decode path).
hipError_t launch_adapter(const uint16_t* w0, int64_t ldw, const TermPtrs& t,
                          int64_t N, int64_t M, int64_t R, const void* x,
                          int64_t T, int64_t ldx, void* y, int y_dtype,
                          int64_t ldy, void* ws, hipStream_t s);

// The head of every workspace carries the decode path's stage-1 -> stage-2
// handoff: 256 bytes of counters, then kSyncSlots producer counters, each in
// its own 256-byte slot (counters packed into a few cache lines made every
// handoff 2-3 us slower).  It is zero before first use and every call leaves
// it zero; no path keeps scratch there.
constexpr size_t kSyncSlots = 64;
constexpr size_t kSyncStride = 64;  // 4-byte words between slots (256 B)
constexpr size_t kWsHeadBytes = 256 + 4 * kSyncSlots * kSyncStride;
static_assert(kWsHeadBytes == DBF_WS_HEAD_BYTES, "workspace head size");

// Row stride (floats) of the rank-R intermediate in the workspace.
inline int64_t ws_rstride(int64_t R) { return (R + 63) / 64 * 64; }

}  // namespace dbf
