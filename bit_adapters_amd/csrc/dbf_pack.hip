// Bit packing of the +-1 factors (one bit per sign, the storage the LoRDBA
// page gives in section 2, "Eficiencia de Armazenamento").  Layout in
// include/dbf.h.  One thread produces one output word, so every word of the
// padded buffer is written exactly once and padding bits come out 0.
#include "dbf_internal.h"

namespace dbf {
namespace {

template <int DT>
__device__ __forceinline__ bool nonneg(const void* src, int64_t i) {
  if constexpr (DT == DBF_I8) {
    return static_cast<const int8_t*>(src)[i] >= 0;
  } else if constexpr (DT == DBF_F32) {
    return static_cast<const float*>(src)[i] >= 0.0f;  // NaN -> false
  } else if constexpr (DT == DBF_BF16) {
    return bf16_bits_to_f32(static_cast<const uint16_t*>(src)[i]) >= 0.0f;
  } else {
    return f16_bits_to_f32(static_cast<const uint16_t*>(src)[i]) >= 0.0f;
  }
}

template <int DT>
__global__ void __launch_bounds__(256)
pack_kernel(const void* __restrict__ src, int64_t rows, int64_t K, int64_t ld,
            uint32_t* __restrict__ out, int64_t nwords, int kw, int64_t nkb) {
  const int64_t widx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (widx >= nwords) return;
  const int64_t tile_words = static_cast<int64_t>(kTileRows) * kw;
  const int64_t tile = widx / tile_words;
  const int64_t in_tile = widx - tile * tile_words;
  const int64_t rt = tile / nkb, kb = tile - rt * nkb;
  const int64_t r = rt * kTileRows + in_tile / kw;
  const int64_t w = in_tile % kw;
  const int64_t k0 = kb * 32 * kw + 32 * w;
  uint32_t word = 0;
  if (r < rows) {
    const int64_t base = r * ld;
    const int64_t kend = K - k0 < 32 ? K - k0 : 32;
    for (int64_t j = 0; j < kend; ++j)
      word |= static_cast<uint32_t>(nonneg<DT>(src, base + k0 + j)) << j;
  }
  out[widx] = word;
}

__global__ void __launch_bounds__(256)
unpack_kernel(const uint32_t* __restrict__ packed, int64_t rows, int64_t K,
              int8_t* __restrict__ dst, int64_t ld, int64_t nwords, int kw,
              int64_t nkb) {
  const int64_t widx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (widx >= nwords) return;
  const int64_t tile_words = static_cast<int64_t>(kTileRows) * kw;
  const int64_t tile = widx / tile_words;
  const int64_t in_tile = widx - tile * tile_words;
  const int64_t rt = tile / nkb, kb = tile - rt * nkb;
  const int64_t r = rt * kTileRows + in_tile / kw;
  const int64_t w = in_tile % kw;
  const int64_t k0 = kb * 32 * kw + 32 * w;
  if (r >= rows || k0 >= K) return;
  const uint32_t word = packed[widx];
  const int64_t kend = K - k0 < 32 ? K - k0 : 32;
  int8_t* o = dst + r * ld + k0;
  for (int64_t j = 0; j < kend; ++j) o[j] = ((word >> j) & 1u) ? 1 : -1;
}

// The packed layout of S^T (K rows x `rows` columns) from that of S (rows x
// K), one output word per thread: output row c, word w of K-block kb holds
// columns 32 (kw' kb + w) .. + 31 of row c of S^T, i.e. bit (c) of input
// rows r0 .. r0 + 31.  Padding bits come out 0.
__global__ void __launch_bounds__(256)
transpose_kernel(const uint32_t* __restrict__ in, int64_t rows, int64_t K,
                 uint32_t* __restrict__ out, int64_t nwords_out, int kw_in, int64_t nkb_in,
                 int kw_out, int64_t nkb_out) {
  const int64_t widx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (widx >= nwords_out) return;
  const int64_t tile_words = static_cast<int64_t>(kTileRows) * kw_out;
  const int64_t tile = widx / tile_words;
  const int64_t in_tile = widx - tile * tile_words;
  const int64_t rt = tile / nkb_out, kb = tile - rt * nkb_out;
  const int64_t c = rt * kTileRows + in_tile / kw_out;  // row of S^T = column of S
  const int64_t w = in_tile % kw_out;
  const int64_t r0 = kb * 32 * kw_out + 32 * w;       // first row of S in this word
  uint32_t word = 0;
  if (c < K) {
    // column c of S sits in K-block c / (32 kw_in), word (c % (32 kw_in)) / 32, bit c % 32
    const int64_t ckb = c / (32 * kw_in);
    const int64_t cw = (c % (32 * kw_in)) / 32;
    const int cb = static_cast<int>(c % 32);
    const int64_t rend = rows - r0 < 32 ? rows - r0 : 32;
    for (int64_t j = 0; j < rend; ++j) {
      const int64_t r = r0 + j;
      const uint32_t src = in[((r / kTileRows) * nkb_in + ckb) * kTileRows * kw_in +
                              (r % kTileRows) * kw_in + cw];
      word |= ((src >> cb) & 1u) << j;
    }
  }
  out[widx] = word;
}

}  // namespace

hipError_t launch_transpose_packed(const uint32_t* packed, int64_t rows, int64_t k,
                                   uint32_t* out, hipStream_t s) {
  const int64_t nwords = layout_words(k, rows);
  const dim3 grid(static_cast<unsigned>((nwords + 255) / 256));
  transpose_kernel<<<grid, 256, 0, s>>>(packed, rows, k, out, nwords,
                                        static_cast<int>(layout_kw(k)), layout_nkb(k),
                                        static_cast<int>(layout_kw(rows)), layout_nkb(rows));
  return hipGetLastError();
}

hipError_t launch_pack(const void* src, int src_dtype, int64_t rows, int64_t k,
                       int64_t ld, uint32_t* packed, hipStream_t s) {
  const int64_t nwords = layout_words(rows, k);
  const int kw = static_cast<int>(layout_kw(k));
  const int64_t nkb = layout_nkb(k);
  const dim3 grid(static_cast<unsigned>((nwords + 255) / 256));
  switch (src_dtype) {
    case DBF_I8:
      pack_kernel<DBF_I8><<<grid, 256, 0, s>>>(src, rows, k, ld, packed, nwords, kw, nkb);
      break;
    case DBF_F16:
      pack_kernel<DBF_F16><<<grid, 256, 0, s>>>(src, rows, k, ld, packed, nwords, kw, nkb);
      break;
    case DBF_BF16:
      pack_kernel<DBF_BF16><<<grid, 256, 0, s>>>(src, rows, k, ld, packed, nwords, kw, nkb);
      break;
    default:
      pack_kernel<DBF_F32><<<grid, 256, 0, s>>>(src, rows, k, ld, packed, nwords, kw, nkb);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_unpack(const uint32_t* packed, int64_t rows, int64_t k,
                         int8_t* dst, int64_t ld, hipStream_t s) {
  const int64_t nwords = layout_words(rows, k);
  const int kw = static_cast<int>(layout_kw(k));
  const int64_t nkb = layout_nkb(k);
  const dim3 grid(static_cast<unsigned>((nwords + 255) / 256));
  unpack_kernel<<<grid, 256, 0, s>>>(packed, rows, k, dst, ld, nwords, kw, nkb);
  return hipGetLastError();
}

}  // namespace dbf
