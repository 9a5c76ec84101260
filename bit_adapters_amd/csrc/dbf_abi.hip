// extern "C" boundary of libdbf: argument validation (before any HIP call),
// the gfx950 device check, path choice and dispatch to the kernels.
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "dbf_internal.h"
#include "dbf_lut.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned2(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 1u) == 0; }

// DBF_PATH_AUTO for the double-binary layer: the decode kernel while T <= 4
// or its sign work, n_terms * ceil(T / 4) * R * (N + M) sign lookups (every
// 4-token block runs both products of every term), is at most
// kAutoDecodeWork; else the MFMA products, whose cost at these token counts
// is nearly flat.  Measured, decode vs MFMA, each path forced (us per call):
//   512 x 512, R 256: decode faster through 64 tokens (12.0 vs 20.7);
//   4096 x 4096, R 2048: faster through 16 tokens (20.3 vs 25.1), slower
//     from 20 (26.9 vs 26.1, sign work 8.4e7);
//   11008 x 4096, R 2048, three terms: faster at 4 tokens (31.3 vs 32.7),
//     slower from 5 (45.7 vs 32.7);
//   8192 x 8192, R 6144: faster at 4 tokens (28.6 vs 33.2), slower at 8
//     (46.4 vs 33.7).
// The boolean kernels (one product each, over a full N x M sign matrix):
// decode while its launch has one token block (up to 2 tokens) or K times
// its token blocks (of 1, 2 or 4 tokens) is at most 4.  Measured: two
// 4096 x 4096 kernels, decode faster through 4 tokens (14.8 vs 18.3 us),
// within 3% at 6 and 8 (17.8 vs 18.4, 18.1 vs 18.4 us); three 11008 x 4096
// kernels, faster through 2 tokens (23.1 vs 28.2 us), slower from 3 (33.8
// vs 28.3 us).
constexpr double kAutoDecodeWork = 8.0e7;
constexpr int64_t kAutoBoolDecodeBlocks = 4;

int resolve_path(int path, int64_t T, int n_terms, int64_t blocks) {
  if (path != DBF_PATH_AUTO) return path;
  const bool decode = T <= 4 || n_terms * ((T + 3) / 4) <= blocks;
  return decode ? DBF_PATH_DECODE : DBF_PATH_MFMA;
}

int resolve_bool_path(int path, int64_t T, int n_kernels) {
  if (path != DBF_PATH_AUTO) return path;
  const int64_t tb = dbf::lut::pick_tb(T);
  const int64_t blocks = (T + tb - 1) / tb;
  return blocks == 1 || n_kernels * blocks <= kAutoBoolDecodeBlocks ? DBF_PATH_DECODE
                                                                    : DBF_PATH_MFMA;
}

int resolve_dbf_path(int path, int64_t N, int64_t M, int64_t R, int64_t T, int n_terms) {
  if (path != DBF_PATH_AUTO) return path;
  const double work = static_cast<double>(n_terms) * static_cast<double>((T + 3) / 4) *
                      static_cast<double>(R) * (static_cast<double>(N) + static_cast<double>(M));
  return T <= 4 || work <= kAutoDecodeWork ? DBF_PATH_DECODE : DBF_PATH_MFMA;
}

constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return fail(DBF_EDEVICE, "no HIP device is current");
  if (dev < kMaxDevices) {
    const int st = g_dev_state[dev].load(std::memory_order_relaxed);
    if (st == 1) return DBF_OK;
    if (st == 2) return fail(DBF_EDEVICE, "device %d is not gfx950", dev);
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
    return fail(DBF_EDEVICE, "cannot query device %d", dev);
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_dev_state[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  if (!ok) return fail(DBF_EDEVICE, "device %d is %s, not gfx950", dev, prop.gcnArchName);
  return DBF_OK;
}

int launched(hipError_t e) {
  if (e != hipSuccess) return fail(DBF_ELAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
  g_err[0] = '\0';
  return DBF_OK;
}

bool out_dtype_ok(int dt) { return dt == DBF_F32 || dt == DBF_BF16 || dt == DBF_F16; }

// Shared validation of the term array (packed factors + scales).
int check_terms(const dbf_term* terms, int n_terms, bool need_gamma,
                bool need_ab) {
  if (!terms) return fail(DBF_EINVAL, "terms is NULL");
  if (n_terms < 1 || n_terms > DBF_MAX_TERMS)
    return fail(DBF_EINVAL, "n_terms %d outside 1..%d", n_terms, DBF_MAX_TERMS);
  for (int i = 0; i < n_terms; ++i) {
    const dbf_term& t = terms[i];
    if (!t.b1 || !t.b2) return fail(DBF_EINVAL, "term %d: packed factor is NULL", i);
    if (!aligned16(t.b1) || !aligned16(t.b2))
      return fail(DBF_EALIGN, "term %d: packed factor not 16-byte aligned", i);
    if (need_ab && (!t.alpha || !t.beta))
      return fail(DBF_EINVAL, "term %d: alpha/beta is NULL", i);
    if (need_gamma && !t.gamma) return fail(DBF_EINVAL, "term %d: gamma is NULL", i);
    if ((t.alpha && !aligned2(t.alpha)) || (t.beta && !aligned2(t.beta)) ||
        (t.gamma && !aligned2(t.gamma)))
      return fail(DBF_EALIGN, "term %d: a scale vector is not 2-byte aligned", i);
  }
  return DBF_OK;
}

dbf::TermPtrs to_ptrs(const dbf_term* terms, int n_terms) {
  dbf::TermPtrs p{};
  p.n = n_terms;
  for (int i = 0; i < n_terms; ++i) {
    p.b1[i] = terms[i].b1;
    p.b2[i] = terms[i].b2;
    p.alpha[i] = static_cast<const uint16_t*>(terms[i].alpha);
    p.beta[i] = static_cast<const uint16_t*>(terms[i].beta);
    p.gamma[i] = static_cast<const uint16_t*>(terms[i].gamma);
  }
  return p;
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return DBF_OK;
  if (!ws) return fail(DBF_EWORKSPACE, "workspace of %zu bytes needed, got NULL", need);
  if (ws_bytes < need)
    return fail(DBF_EWORKSPACE, "workspace of %zu bytes needed, got %zu", need, ws_bytes);
  if (!aligned16(ws)) return fail(DBF_EALIGN, "workspace not 16-byte aligned");
  return DBF_OK;
}

int linear_forward(const dbf_term* terms, int n_terms, int64_t N, int64_t M, int64_t R,
                   const void* x, int x_dtype, int64_t T, int64_t ldx, void* y, int y_dtype,
                   int64_t ldy, int accumulate, void* ws, size_t ws_bytes, bool noalloc, int path,
                   void* stream);

}  // namespace

// ---- scratch of dbf_linear_forward_noalloc --------------------------------
// The workspace of the allocation-free entry point: a fixed array in the
// library's code object, so each device that loads the library holds its own
// copy until the process ends.  Its first DBF_WS_HEAD_BYTES are the decode
// path's handoff counters: zero at load, cleared once more at set-up, and
// left zero by every call.
static __device__ __align__(256) unsigned char scratch[DBF_NOALLOC_SCRATCH_BYTES];

namespace {

__global__ void __launch_bounds__(256) zero_words_kernel(uint32_t* p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device

// The current device's address of `scratch`, looked up (hipGetSymbolAddress)
// and its head cleared on the first call on that device.  In host code the
// array's name is only a stand-in for the symbol; kernels get this address.
int scratch_address(hipStream_t s, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return fail(DBF_EDEVICE, "no HIP device is current");
  if (dev >= kMaxDevices) return fail(DBF_EDEVICE, "device %d is past the %d this library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(DBF_ELAUNCH, "looking up the scratch array on device %d failed: %s", dev,
                  hipGetErrorString(e));
    // a fill kernel rather than a memset node, so a first call under graph
    // capture records nothing that replays differently
    constexpr int64_t kHeadWords = DBF_WS_HEAD_BYTES / 4;
    zero_words_kernel<<<dim3(static_cast<unsigned>((kHeadWords + 255) / 256)), 256, 0, s>>>(
        static_cast<uint32_t*>(ptr), kHeadWords);
    const hipError_t le = hipGetLastError();
    if (le != hipSuccess)
      return fail(DBF_ELAUNCH, "clearing the scratch head failed: %s", hipGetErrorString(le));
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return DBF_OK;
}

}  // namespace

extern "C" {

int dbf_abi_version(void) { return DBF_ABI_VERSION; }
int dbf_layout_version(void) { return DBF_LAYOUT_VERSION; }
const char* dbf_last_error(void) { return g_err; }

int dbf_workspace_check(void* ws, void* stream) {
  if (!ws) return fail(DBF_EINVAL, "workspace is NULL");
  if (!aligned16(ws)) return fail(DBF_EALIGN, "workspace not 16-byte aligned");
  // ctr[2] (a wait gave up) and ctr[3] (an adapter index out of range) of
  // the handoff head (dbf_lut.h, Sync)
  unsigned flag[2] = {0, 0};
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(flag, static_cast<unsigned char*>(ws) + 8, sizeof(flag),
                                hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(DBF_ELAUNCH, "reading the workspace failed: %s", hipGetErrorString(e));
  if (flag[0] == 0 && flag[1] == 0) return DBF_OK;
  e = hipMemsetAsync(ws, 0, DBF_WS_HEAD_BYTES, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(DBF_ELAUNCH, "clearing the workspace failed: %s", hipGetErrorString(e));
  if (flag[0] != 0)
    return fail(DBF_ESTALLED, "a handoff wait gave up; the outputs of the calls since the last check are not valid");
  return fail(DBF_EINVAL, "an adapter index was outside [-1, n_adapters); those tokens got the base alone");
}

size_t dbf_packed_bytes(int64_t rows, int64_t k) {
  if (rows <= 0 || k <= 0) return 0;
  return static_cast<size_t>(dbf::layout_words(rows, k)) * 4u;
}

int dbf_pack(const void* src, int src_dtype, int64_t rows, int64_t k,
             int64_t ld, uint32_t* packed, void* stream) {
  if (rows < 0 || k < 0) return fail(DBF_EINVAL, "negative size");
  if (src_dtype != DBF_I8 && src_dtype != DBF_F16 && src_dtype != DBF_BF16 &&
      src_dtype != DBF_F32)
    return fail(DBF_EDTYPE, "pack source dtype %d unsupported", src_dtype);
  if (rows == 0 || k == 0) return DBF_OK;
  if (!src || !packed) return fail(DBF_EINVAL, "NULL pointer");
  if (ld < k) return fail(DBF_EINVAL, "ld %lld < k %lld", (long long)ld, (long long)k);
  if (!aligned16(packed)) return fail(DBF_EALIGN, "packed buffer not 16-byte aligned");
  const int d = check_device();
  if (d != DBF_OK) return d;
  return launched(dbf::launch_pack(src, src_dtype, rows, k, ld, packed,
                                   static_cast<hipStream_t>(stream)));
}

int dbf_unpack(const uint32_t* packed, int64_t rows, int64_t k, int8_t* dst,
               int64_t ld, void* stream) {
  if (rows < 0 || k < 0) return fail(DBF_EINVAL, "negative size");
  if (rows == 0 || k == 0) return DBF_OK;
  if (!packed || !dst) return fail(DBF_EINVAL, "NULL pointer");
  if (ld < k) return fail(DBF_EINVAL, "ld %lld < k %lld", (long long)ld, (long long)k);
  if (!aligned16(packed)) return fail(DBF_EALIGN, "packed buffer not 16-byte aligned");
  const int d = check_device();
  if (d != DBF_OK) return d;
  return launched(dbf::launch_unpack(packed, rows, k, dst, ld,
                                     static_cast<hipStream_t>(stream)));
}

size_t dbf_workspace_bytes(int64_t N, int64_t M, int64_t R, int n_terms,
                           int64_t T, int path) {
  if (N <= 0 || M <= 0 || R <= 0 || n_terms <= 0 || T <= 0) return 0;
  if (resolve_dbf_path(path, N, M, R, T, n_terms) == DBF_PATH_MFMA)
    return dbf::mfma_ws_bytes(N, M, R, n_terms, T);
  return dbf::decode_ws_bytes(N, M, R, n_terms, T);
}

int dbf_linear_forward(const dbf_term* terms, int n_terms, int64_t N,
                       int64_t M, int64_t R, const void* x, int x_dtype,
                       int64_t T, int64_t ldx, void* y, int y_dtype,
                       int64_t ldy, int accumulate, void* ws, size_t ws_bytes,
                       int path, void* stream) {
  return linear_forward(terms, n_terms, N, M, R, x, x_dtype, T, ldx, y, y_dtype, ldy, accumulate,
                        ws, ws_bytes, false, path, stream);
}

int dbf_linear_forward_noalloc(const dbf_term* terms, int n_terms, int64_t N, int64_t M,
                               int64_t R, const void* x, int x_dtype, int64_t T, int64_t ldx,
                               void* y, int y_dtype, int64_t ldy, int accumulate, int path,
                               void* stream) {
  return linear_forward(terms, n_terms, N, M, R, x, x_dtype, T, ldx, y, y_dtype, ldy, accumulate,
                        nullptr, 0, true, path, stream);
}

}  // extern "C"

namespace {

// dbf_linear_forward and dbf_linear_forward_noalloc: the same validation and
// kernels; the second takes its workspace from the library's scratch array.
int linear_forward(const dbf_term* terms, int n_terms, int64_t N, int64_t M, int64_t R,
                   const void* x, int x_dtype, int64_t T, int64_t ldx, void* y, int y_dtype,
                   int64_t ldy, int accumulate, void* ws, size_t ws_bytes, bool noalloc, int path,
                   void* stream) {
  int e = check_terms(terms, n_terms, true, true);
  if (e != DBF_OK) return e;
  if (N < 1 || M < 1 || R < 1) return fail(DBF_EINVAL, "N, M, R must be >= 1");
  if (T < 0) return fail(DBF_EINVAL, "T < 0");
  if (x_dtype != DBF_BF16 && x_dtype != DBF_F16)
    return fail(DBF_EDTYPE, "x dtype %d unsupported (bf16 or f16)", x_dtype);
  if (!out_dtype_ok(y_dtype)) return fail(DBF_EDTYPE, "y dtype %d unsupported", y_dtype);
  if (accumulate != 0 && accumulate != 1) return fail(DBF_EINVAL, "accumulate must be 0 or 1");
  if (path != DBF_PATH_AUTO && path != DBF_PATH_DECODE && path != DBF_PATH_MFMA)
    return fail(DBF_EINVAL, "unknown path %d", path);
  if (T == 0) return DBF_OK;
  if (!x || !y) return fail(DBF_EINVAL, "x or y is NULL");
  if (ldx < M) return fail(DBF_EINVAL, "ldx %lld < M %lld", (long long)ldx, (long long)M);
  if (ldy < N) return fail(DBF_EINVAL, "ldy %lld < N %lld", (long long)ldy, (long long)N);
  if (!aligned16(x) || !aligned16(y)) return fail(DBF_EALIGN, "x or y not 16-byte aligned");
  const int p = resolve_dbf_path(path, N, M, R, T, n_terms);
  const size_t need = dbf_workspace_bytes(N, M, R, n_terms, T, p);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (noalloc) {
    if (need > DBF_NOALLOC_SCRATCH_BYTES)
      return fail(DBF_EWORKSPACE,
                  "this call needs %zu bytes of workspace, more than the %zu of the "
                  "library's scratch; use dbf_linear_forward with a workspace",
                  need, static_cast<size_t>(DBF_NOALLOC_SCRATCH_BYTES));
    e = check_device();
    if (e != DBF_OK) return e;
    e = scratch_address(s, &ws);
    if (e != DBF_OK) return e;
  } else {
    e = check_ws(ws, ws_bytes, need);
    if (e != DBF_OK) return e;
    e = check_device();
    if (e != DBF_OK) return e;
  }
  const dbf::TermPtrs tp = to_ptrs(terms, n_terms);
  if (p == DBF_PATH_MFMA)
    return launched(dbf::launch_mfma(tp, N, M, R, x, x_dtype, T, ldx, y, y_dtype,
                                     ldy, accumulate, ws, s));
  return launched(dbf::launch_decode(tp, N, M, R, x, x_dtype, T, ldx, y, y_dtype,
                                     ldy, accumulate, ws, s));
}

}  // namespace

extern "C" {

size_t dbf_svid_workspace_bytes(int64_t N, int64_t M) {
  if (N <= 0 || M <= 0) return 0;
  return dbf::svid_ws_bytes(N, M);
}

int dbf_svid_extract(const void* w, int w_dtype, int64_t N, int64_t M, int64_t ldw, int n_kernels,
                     const dbf_bool_kernel_out* kernels, int iters, float* residual_sq, void* ws,
                     size_t ws_bytes, void* stream) {
  if (N < 1 || M < 1) return fail(DBF_EINVAL, "N, M must be >= 1");
  if (w_dtype != DBF_F32 && w_dtype != DBF_BF16 && w_dtype != DBF_F16)
    return fail(DBF_EDTYPE, "w dtype %d unsupported (f32, bf16 or f16)", w_dtype);
  if (!w) return fail(DBF_EINVAL, "w is NULL");
  if (ldw < M) return fail(DBF_EINVAL, "ldw %lld < M %lld", (long long)ldw, (long long)M);
  if (reinterpret_cast<uintptr_t>(w) % (w_dtype == DBF_F32 ? 4u : 2u) != 0)
    return fail(DBF_EALIGN, "w not aligned to its element");
  if (!kernels) return fail(DBF_EINVAL, "kernels is NULL");
  if (n_kernels < 1 || n_kernels > DBF_MAX_TERMS)
    return fail(DBF_EINVAL, "n_kernels %d outside 1..%d", n_kernels, DBF_MAX_TERMS);
  if (iters < 1 || iters > 1000) return fail(DBF_EINVAL, "iters %d outside 1..1000", iters);
  uint32_t* wb[DBF_MAX_TERMS];
  uint16_t* sin[DBF_MAX_TERMS];
  uint16_t* sout[DBF_MAX_TERMS];
  for (int k = 0; k < n_kernels; ++k) {
    const dbf_bool_kernel_out& o = kernels[k];
    if (!o.w || !o.s_in || !o.s_out) return fail(DBF_EINVAL, "kernel %d: an output is NULL", k);
    if (!aligned16(o.w)) return fail(DBF_EALIGN, "kernel %d: packed signs not 16-byte aligned", k);
    if (!aligned2(o.s_in) || !aligned2(o.s_out))
      return fail(DBF_EALIGN, "kernel %d: a scale vector is not 2-byte aligned", k);
    wb[k] = o.w;
    sin[k] = static_cast<uint16_t*>(o.s_in);
    sout[k] = static_cast<uint16_t*>(o.s_out);
  }
  if (residual_sq && (reinterpret_cast<uintptr_t>(residual_sq) & 3u))
    return fail(DBF_EALIGN, "residual_sq not 4-byte aligned");
  int e = check_ws(ws, ws_bytes, dbf_svid_workspace_bytes(N, M));
  if (e != DBF_OK) return e;
  e = check_device();
  if (e != DBF_OK) return e;
  return launched(dbf::launch_svid(w, w_dtype, N, M, ldw, n_kernels, wb, sin, sout, iters,
                                   residual_sq, ws, static_cast<hipStream_t>(stream)));
}

int dbf_transpose_packed(const uint32_t* packed, int64_t rows, int64_t k, uint32_t* out,
                         void* stream) {
  if (rows < 0 || k < 0) return fail(DBF_EINVAL, "negative size");
  if (rows == 0 || k == 0) return DBF_OK;
  if (!packed || !out) return fail(DBF_EINVAL, "NULL pointer");
  if (!aligned16(packed) || !aligned16(out)) return fail(DBF_EALIGN, "packed buffer not 16-byte aligned");
  const int d = check_device();
  if (d != DBF_OK) return d;
  return launched(dbf::launch_transpose_packed(packed, rows, k, out, static_cast<hipStream_t>(stream)));
}

size_t dbf_backward_workspace_bytes(int64_t N, int64_t M, int64_t R, int n_terms, int64_t T,
                                    int path) {
  if (N <= 0 || M <= 0 || R <= 0 || n_terms <= 0 || T <= 0) return 0;
  return dbf::backward_ws_bytes(N, M, R, n_terms, T, resolve_path(path, T, 1, kAutoBoolDecodeBlocks));
}

int dbf_linear_backward(const dbf_term* terms, const dbf_term_t* tterms, int n_terms, int64_t N,
                        int64_t M, int64_t R, const void* x, int x_dtype, int64_t ldx,
                        const void* dy, int dy_dtype, int64_t lddy, int64_t T, void* dx,
                        int dx_dtype, int64_t lddx, float* dalpha, float* dbeta, float* dgamma,
                        void* ws, size_t ws_bytes, int path, void* stream) {
  int e = check_terms(terms, n_terms, true, true);
  if (e != DBF_OK) return e;
  if (!tterms) return fail(DBF_EINVAL, "tterms is NULL");
  for (int i = 0; i < n_terms; ++i) {
    if (!tterms[i].b1t || !tterms[i].b2t) return fail(DBF_EINVAL, "term %d: transposed factor is NULL", i);
    if (!aligned16(tterms[i].b1t) || !aligned16(tterms[i].b2t))
      return fail(DBF_EALIGN, "term %d: transposed factor not 16-byte aligned", i);
  }
  if (N < 1 || M < 1 || R < 1) return fail(DBF_EINVAL, "N, M, R must be >= 1");
  if (T < 0) return fail(DBF_EINVAL, "T < 0");
  if (x_dtype != DBF_BF16 && x_dtype != DBF_F16)
    return fail(DBF_EDTYPE, "x dtype %d unsupported (bf16 or f16)", x_dtype);
  if (dy_dtype != DBF_BF16 && dy_dtype != DBF_F16 && dy_dtype != DBF_F32)
    return fail(DBF_EDTYPE, "dy dtype %d unsupported", dy_dtype);
  if (dx && !out_dtype_ok(dx_dtype)) return fail(DBF_EDTYPE, "dx dtype %d unsupported", dx_dtype);
  if (path != DBF_PATH_AUTO && path != DBF_PATH_DECODE && path != DBF_PATH_MFMA)
    return fail(DBF_EINVAL, "unknown path %d", path);
  if (T == 0) return DBF_OK;
  if (!x || !dy) return fail(DBF_EINVAL, "x or dy is NULL");
  if (ldx < M) return fail(DBF_EINVAL, "ldx %lld < M %lld", (long long)ldx, (long long)M);
  if (lddy < N) return fail(DBF_EINVAL, "lddy %lld < N %lld", (long long)lddy, (long long)N);
  if (dx && lddx < M) return fail(DBF_EINVAL, "lddx %lld < M %lld", (long long)lddx, (long long)M);
  if (!aligned16(x) || !aligned16(dy) || (dx && !aligned16(dx)))
    return fail(DBF_EALIGN, "x, dy or dx not 16-byte aligned");
  if ((dalpha && (reinterpret_cast<uintptr_t>(dalpha) & 3u)) ||
      (dbeta && (reinterpret_cast<uintptr_t>(dbeta) & 3u)) ||
      (dgamma && (reinterpret_cast<uintptr_t>(dgamma) & 3u)))
    return fail(DBF_EALIGN, "a scale gradient is not 4-byte aligned");
  const int p = resolve_path(path, T, 1, kAutoBoolDecodeBlocks);
  e = check_ws(ws, ws_bytes, dbf_backward_workspace_bytes(N, M, R, n_terms, T, p));
  if (e != DBF_OK) return e;
  e = check_device();
  if (e != DBF_OK) return e;
  const dbf::TermPtrs tp = to_ptrs(terms, n_terms);
  const uint32_t* b1t[DBF_MAX_TERMS];
  const uint32_t* b2t[DBF_MAX_TERMS];
  for (int i = 0; i < n_terms; ++i) {
    b1t[i] = tterms[i].b1t;
    b2t[i] = tterms[i].b2t;
  }
  return launched(dbf::launch_backward(tp, b1t, b2t, N, M, R, x, x_dtype, ldx, dy, dy_dtype, lddy,
                                       T, dx, dx_dtype, lddx, dalpha, dbeta, dgamma, p, ws,
                                       static_cast<hipStream_t>(stream)));
}

int lordba_multi_adapter_forward(const void* w0, int64_t ldw, const dbf_term* adapters,
                                 int n_adapters, int64_t N, int64_t M, int64_t R,
                                 const int32_t* adapter_idx, const void* x, int64_t T, int64_t ldx,
                                 void* y, int y_dtype, int64_t ldy, void* ws, size_t ws_bytes,
                                 void* stream) {
  if (n_adapters < 1 || n_adapters > DBF_MAX_ADAPTERS)
    return fail(DBF_EINVAL, "n_adapters %d outside 1..%d", n_adapters, DBF_MAX_ADAPTERS);
  if (!adapters) return fail(DBF_EINVAL, "adapters is NULL");
  for (int a = 0; a < n_adapters; ++a) {
    const int e = check_terms(adapters + a, 1, true, true);
    if (e != DBF_OK) return e;
  }
  if (!w0) return fail(DBF_EINVAL, "w0 is NULL");
  if (N < 1 || M < 1 || R < 1) return fail(DBF_EINVAL, "N, M, R must be >= 1");
  if (T < 0) return fail(DBF_EINVAL, "T < 0");
  if (ldw < M) return fail(DBF_EINVAL, "ldw %lld < M %lld", (long long)ldw, (long long)M);
  if (!out_dtype_ok(y_dtype)) return fail(DBF_EDTYPE, "y dtype %d unsupported", y_dtype);
  if (!aligned16(w0)) return fail(DBF_EALIGN, "w0 not 16-byte aligned");
  if (T == 0) return DBF_OK;
  if (!x || !y || !adapter_idx) return fail(DBF_EINVAL, "x, y or adapter_idx is NULL");
  if (ldx < M) return fail(DBF_EINVAL, "ldx %lld < M %lld", (long long)ldx, (long long)M);
  if (ldy < N) return fail(DBF_EINVAL, "ldy %lld < N %lld", (long long)ldy, (long long)N);
  if (!aligned16(x) || !aligned16(y)) return fail(DBF_EALIGN, "x or y not 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(adapter_idx) & 3u)
    return fail(DBF_EALIGN, "adapter_idx not 4-byte aligned");
  int e = check_ws(ws, ws_bytes, dbf_workspace_bytes(N, M, R, 1, T, DBF_PATH_DECODE));
  if (e != DBF_OK) return e;
  e = check_device();
  if (e != DBF_OK) return e;
  dbf::TermPtrs tp[DBF_MAX_ADAPTERS];
  for (int a = 0; a < n_adapters; ++a) tp[a] = to_ptrs(adapters + a, 1);
  return launched(dbf::launch_multi_adapter(static_cast<const uint16_t*>(w0), ldw, tp, n_adapters,
                                            N, M, R, adapter_idx, x, T, ldx, y, y_dtype, ldy, ws,
                                            static_cast<hipStream_t>(stream)));
}

size_t dbf_bool_workspace_bytes(int64_t N, int64_t M, int n_kernels, int64_t T, int path) {
  if (N <= 0 || M <= 0 || n_kernels <= 0 || T <= 0) return 0;
  if (resolve_bool_path(path, T, n_kernels) == DBF_PATH_MFMA)
    return dbf::mfma_bool_ws_bytes(N, M, n_kernels, T);
  return dbf::decode_ws_bytes(N, M, N, n_kernels, T);
}

int dbf_bool_forward(const dbf_bool_kernel* kernels, int n_kernels, int64_t N, int64_t M,
                     const void* x, int x_dtype, int64_t T, int64_t ldx, void* y,
                     int y_dtype, int64_t ldy, int accumulate, void* ws, size_t ws_bytes,
                     int path, void* stream) {
  if (!kernels) return fail(DBF_EINVAL, "kernels is NULL");
  if (n_kernels < 1 || n_kernels > DBF_MAX_TERMS)
    return fail(DBF_EINVAL, "n_kernels %d outside 1..%d", n_kernels, DBF_MAX_TERMS);
  for (int i = 0; i < n_kernels; ++i) {
    const dbf_bool_kernel& k = kernels[i];
    if (!k.w || !k.s_in || !k.s_out) return fail(DBF_EINVAL, "kernel %d: a pointer is NULL", i);
    if (!aligned16(k.w)) return fail(DBF_EALIGN, "kernel %d: packed signs not 16-byte aligned", i);
    if (!aligned2(k.s_in) || !aligned2(k.s_out))
      return fail(DBF_EALIGN, "kernel %d: a scale vector is not 2-byte aligned", i);
  }
  if (N < 1 || M < 1) return fail(DBF_EINVAL, "N, M must be >= 1");
  if (T < 0) return fail(DBF_EINVAL, "T < 0");
  if (x_dtype != DBF_BF16 && x_dtype != DBF_F16)
    return fail(DBF_EDTYPE, "x dtype %d unsupported (bf16 or f16)", x_dtype);
  if (!out_dtype_ok(y_dtype)) return fail(DBF_EDTYPE, "y dtype %d unsupported", y_dtype);
  if (accumulate != 0 && accumulate != 1) return fail(DBF_EINVAL, "accumulate must be 0 or 1");
  if (path != DBF_PATH_AUTO && path != DBF_PATH_DECODE && path != DBF_PATH_MFMA)
    return fail(DBF_EINVAL, "unknown path %d", path);
  if (T == 0) return DBF_OK;
  if (!x || !y) return fail(DBF_EINVAL, "x or y is NULL");
  if (ldx < M) return fail(DBF_EINVAL, "ldx %lld < M %lld", (long long)ldx, (long long)M);
  if (ldy < N) return fail(DBF_EINVAL, "ldy %lld < N %lld", (long long)ldy, (long long)N);
  if (!aligned16(x) || !aligned16(y)) return fail(DBF_EALIGN, "x or y not 16-byte aligned");
  const int p = resolve_bool_path(path, T, n_kernels);
  int e = check_ws(ws, ws_bytes, dbf_bool_workspace_bytes(N, M, n_kernels, T, p));
  if (e != DBF_OK) return e;
  e = check_device();
  if (e != DBF_OK) return e;
  // the kernels in the roles of the double-binary path's sign matrices and
  // scales: decode uses the stage-1 slots (b2, gamma, beta), MFMA the
  // stage-2 ones (b1, alpha) plus gamma
  dbf::TermPtrs tp{};
  tp.n = n_kernels;
  for (int i = 0; i < n_kernels; ++i) {
    tp.b1[i] = tp.b2[i] = kernels[i].w;
    tp.gamma[i] = static_cast<const uint16_t*>(kernels[i].s_in);
    tp.alpha[i] = tp.beta[i] = static_cast<const uint16_t*>(kernels[i].s_out);
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (p == DBF_PATH_MFMA)
    return launched(dbf::launch_bool_mfma(tp, N, M, x, x_dtype, T, ldx, y, y_dtype, ldy,
                                          accumulate, ws, s));
  return launched(dbf::launch_bool_decode(tp, N, M, x, x_dtype, T, ldx, y, y_dtype, ldy,
                                          accumulate, ws, s));
}

int dbf_linear_forward_i8(const dbf_term* terms, int n_terms, int64_t N,
                          int64_t M, int64_t R, const int8_t* x, int64_t T,
                          int64_t ldx, int32_t* s1, int32_t* s2, void* y,
                          int y_dtype, int64_t ldy, void* ws, size_t ws_bytes,
                          void* stream) {
  int e = check_terms(terms, n_terms, false, false);
  if (e != DBF_OK) return e;
  if (N < 1 || M < 1 || R < 1) return fail(DBF_EINVAL, "N, M, R must be >= 1");
  if (T < 0) return fail(DBF_EINVAL, "T < 0");
  bool beta_null = terms[0].beta == nullptr;
  for (int i = 0; i < n_terms; ++i) {
    if (terms[i].gamma)
      return fail(DBF_EINVAL, "term %d: gamma must be NULL (fold it into x upstream)", i);
    if ((terms[i].beta == nullptr) != beta_null)
      return fail(DBF_EINVAL, "beta must be NULL in all terms or in none");
  }
  if (s2 && !beta_null) return fail(DBF_EINVAL, "s2 needs beta == NULL (beta = 1)");
  if (y && !out_dtype_ok(y_dtype)) return fail(DBF_EDTYPE, "y dtype %d unsupported", y_dtype);
  if (static_cast<double>(M) * 127.0 >= 2147483648.0)
    return fail(DBF_EUNSUPPORTED, "M * 127 does not fit int32");
  if ((s2 || beta_null) && static_cast<double>(R) * static_cast<double>(M) * 127.0 >= 2147483648.0)
    return fail(DBF_EUNSUPPORTED, "R * M * 127 does not fit int32");
  if (T == 0) return DBF_OK;
  if (!x) return fail(DBF_EINVAL, "x is NULL");
  if (ldx < M) return fail(DBF_EINVAL, "ldx %lld < M %lld", (long long)ldx, (long long)M);
  if (y && ldy < N) return fail(DBF_EINVAL, "ldy %lld < N %lld", (long long)ldy, (long long)N);
  if (!aligned16(x) || (y && !aligned16(y)) || (s1 && !aligned16(s1)) ||
      (s2 && !aligned16(s2)))
    return fail(DBF_EALIGN, "x, y, s1 or s2 not 16-byte aligned");
  e = check_ws(ws, ws_bytes, dbf_workspace_bytes(N, M, R, n_terms, T, DBF_PATH_DECODE));
  if (e != DBF_OK) return e;
  e = check_device();
  if (e != DBF_OK) return e;
  return launched(dbf::launch_decode_i8(to_ptrs(terms, n_terms), N, M, R, x, T,
                                        ldx, s1, s2, y, y_dtype, ldy, ws,
                                        static_cast<hipStream_t>(stream)));
}

int lordba_adapter_forward(const void* w0, int64_t ldw, const dbf_term* terms,
                           int n_terms, int64_t N, int64_t M, int64_t R,
                           const void* x, int64_t T, int64_t ldx, void* y,
                           int y_dtype, int64_t ldy, void* ws,
                           size_t ws_bytes, void* stream) {
  if (n_terms < 0 || n_terms > DBF_MAX_TERMS)
    return fail(DBF_EINVAL, "n_terms %d outside 0..%d", n_terms, DBF_MAX_TERMS);
  int e = DBF_OK;
  if (n_terms > 0) {
    e = check_terms(terms, n_terms, true, true);
    if (e != DBF_OK) return e;
    if (R < 1) return fail(DBF_EINVAL, "R must be >= 1");
  }
  if (N < 1 || M < 1) return fail(DBF_EINVAL, "N, M must be >= 1");
  if (T < 0) return fail(DBF_EINVAL, "T < 0");
  if (!out_dtype_ok(y_dtype)) return fail(DBF_EDTYPE, "y dtype %d unsupported", y_dtype);
  if (T == 0) return DBF_OK;
  if (!w0 || !x || !y) return fail(DBF_EINVAL, "w0, x or y is NULL");
  if (ldw < M) return fail(DBF_EINVAL, "ldw %lld < M %lld", (long long)ldw, (long long)M);
  if (ldx < M) return fail(DBF_EINVAL, "ldx %lld < M %lld", (long long)ldx, (long long)M);
  if (ldy < N) return fail(DBF_EINVAL, "ldy %lld < N %lld", (long long)ldy, (long long)N);
  if (!aligned16(w0) || !aligned16(x) || !aligned16(y))
    return fail(DBF_EALIGN, "w0, x or y not 16-byte aligned");
  if (n_terms > 0) {
    e = check_ws(ws, ws_bytes, dbf_workspace_bytes(N, M, R, n_terms, T, DBF_PATH_DECODE));
    if (e != DBF_OK) return e;
  }
  e = check_device();
  if (e != DBF_OK) return e;
  const dbf::TermPtrs tp = n_terms > 0 ? to_ptrs(terms, n_terms) : dbf::TermPtrs{};
  return launched(dbf::launch_adapter(static_cast<const uint16_t*>(w0), ldw, tp, N, M,
                                      n_terms > 0 ? R : 1, x, T, ldx, y, y_dtype, ldy, ws,
                                      static_cast<hipStream_t>(stream)));
}

}  // extern "C"
