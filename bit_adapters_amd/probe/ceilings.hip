// Machine ceilings of one MI355X (gfx950), measured the way the layer's
// kernels use the machine.  Test and measurement infrastructure: nothing in
// libdbf calls it.
//
//   empty     launch cost of an empty kernel, K launches replayed from a HIP
//             graph (per-launch time)
//   read      streaming read of S bytes (16-byte loads, grid-stride), each
//             launch on a different S-byte window of a 1 GiB buffer so the
//             bytes come from HBM, not the 256 MiB MALL or the L2s
//   mfma      v_mfma_f32_32x32x16_f16 issue rate with 8 independent
//             accumulators per wave on every SIMD, operands (a) varied fp16
//             values and (b) +-1, the sign-matrix operand of the layer
//   flag      cross-workgroup visibility: one workgroup stores a flag with a
//             system-scope atomic, a workgroup on another XCD (workgroup ids
//             go round-robin over the 8 XCDs) polls it; both read the 100 MHz
//             constant clock.  The poll is bounded (2^22 rounds).
//
// Output: one line per measurement, "name value unit".
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <vector>

#define CK(x)                                                                    \
  do {                                                                           \
    hipError_t e_ = (x);                                                         \
    if (e_ != hipSuccess) {                                                      \
      std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));        \
      std::exit(1);                                                              \
    }                                                                            \
  } while (0)

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

__global__ void empty_kernel() {}

__global__ void __launch_bounds__(256) read_kernel(const uint4* __restrict__ p, size_t n16,
                                                   unsigned* out) {
  unsigned acc = 0;
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
#pragma unroll 8
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) out[0] = acc;  // keeps the loads; practically never true
}

constexpr int kChains = 8;

__global__ void __launch_bounds__(256) mfma_kernel(int iters, int unit_b, float* out) {
  const unsigned lane = threadIdx.x & 63;
  half8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<_Float16>(0.001f * static_cast<float>((lane * 8 + i) % 97) - 0.05f);
    b[i] = unit_b ? static_cast<_Float16>(((lane >> (i & 3)) & 1) ? 1.f : -1.f)
                  : static_cast<_Float16>(0.002f * static_cast<float>((lane * 5 + 3 * i) % 89) - 0.09f);
  }
  floatx16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  if (s == 123456.f) out[0] = s;  // keeps the MFMAs; practically never true
}

// Workgroup 0 (XCD 0) sets flag[0] after a delay; workgroup `peer` (another
// XCD) polls it.  t[0] = clock just before the store, t[1] = clock when the
// poll saw it, t[2] = 1 if the poll gave up.
__global__ void flag_kernel(unsigned* flag, unsigned long long* t, int peer) {
  if (threadIdx.x != 0) return;
  if (blockIdx.x == 0) {
    const unsigned long long t0 = wall_clock64();
    while (wall_clock64() - t0 < 2000) {}  // 20 us: the peer is polling by now
    const unsigned long long ts = wall_clock64();
    __hip_atomic_store(flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    t[0] = ts;
  } else if (static_cast<int>(blockIdx.x) == peer) {
    unsigned spins = 0;
    while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) == 0u) {
      if (++spins > (1u << 22)) {
        t[2] = 1;
        break;
      }
    }
    t[1] = wall_clock64();
  }
}

static float time_graph(hipGraphExec_t g, hipStream_t s) {
  hipEvent_t a, b;
  CK(hipEventCreate(&a));
  CK(hipEventCreate(&b));
  CK(hipGraphLaunch(g, s));  // warm
  CK(hipStreamSynchronize(s));
  CK(hipEventRecord(a, s));
  CK(hipGraphLaunch(g, s));
  CK(hipEventRecord(b, s));
  CK(hipEventSynchronize(b));
  float ms = 0.f;
  CK(hipEventElapsedTime(&ms, a, b));
  CK(hipEventDestroy(a));
  CK(hipEventDestroy(b));
  return ms;
}

template <class F>
static hipGraphExec_t capture(hipStream_t s, F&& body) {
  hipGraph_t g;
  hipGraphExec_t ge;
  CK(hipStreamBeginCapture(s, hipStreamCaptureModeGlobal));
  body();
  CK(hipStreamEndCapture(s, &g));
  CK(hipGraphInstantiate(&ge, g, nullptr, nullptr, 0));
  CK(hipGraphDestroy(g));
  return ge;
}

int main() {
  hipDeviceProp_t prop;
  CK(hipGetDeviceProperties(&prop, 0));
  std::printf("device %s cus %d\n", prop.gcnArchName, prop.multiProcessorCount);
  const int cus = prop.multiProcessorCount;
  hipStream_t s;
  CK(hipStreamCreate(&s));
  unsigned* sink;
  CK(hipMalloc(&sink, 64));

  {  // empty kernel
    const int K = 1000;
    hipGraphExec_t g = capture(s, [&] {
      for (int i = 0; i < K; ++i) empty_kernel<<<1, 64, 0, s>>>();
    });
    std::printf("empty_kernel_graph %.3f us/launch\n", 1000.f * time_graph(g, s) / K);
    CK(hipGraphExecDestroy(g));
  }

  {  // streaming read
    const size_t total = size_t(1) << 30;
    unsigned char* buf;
    CK(hipMalloc(&buf, total));
    CK(hipMemset(buf, 1, total));
    for (size_t sz : {size_t(2) << 20, size_t(32) << 20, size_t(512) << 20}) {
      const int nwin = static_cast<int>(total / sz);
      const int K = std::max(8, std::min(400, 2 * nwin));
      const unsigned grid = static_cast<unsigned>(std::min<size_t>(sz / 16 / 256, size_t(cus) * 16));
      hipGraphExec_t g = capture(s, [&] {
        for (int i = 0; i < K; ++i)
          read_kernel<<<grid, 256, 0, s>>>(reinterpret_cast<const uint4*>(buf + (i % nwin) * sz), sz / 16, sink);
      });
      const float ms = time_graph(g, s) / K;
      std::printf("read_%zuMiB %.3f us %.1f GB/s\n", sz >> 20, 1000.f * ms, sz / (ms * 1e6));
      CK(hipGraphExecDestroy(g));
    }
    CK(hipFree(buf));
  }

  {  // MFMA issue rate
    const int iters = 4000, wgs = cus * 8;
    for (int unit_b = 0; unit_b < 2; ++unit_b) {
      hipGraphExec_t g = capture(s, [&] { mfma_kernel<<<wgs, 256, 0, s>>>(iters, unit_b, reinterpret_cast<float*>(sink)); });
      const float ms = time_graph(g, s);
      const double flops = double(wgs) * 4 * iters * kChains * 32.0 * 32.0 * 16.0 * 2.0;
      std::printf("mfma_f32_32x32x16_f16_%s %.1f TFLOP/s\n", unit_b ? "pm1" : "varied", flops / (ms * 1e9));
      CK(hipGraphExecDestroy(g));
    }
  }

  {  // cross-XCD flag visibility
    unsigned* flag;
    unsigned long long* t;
    CK(hipMalloc(&flag, 256));
    CK(hipMalloc(&t, 3 * sizeof(unsigned long long)));
    std::vector<double> lat;
    for (int rep = 0; rep < 20; ++rep) {
      CK(hipMemset(flag, 0, 256));
      CK(hipMemset(t, 0, 3 * sizeof(unsigned long long)));
      flag_kernel<<<8, 64, 0, s>>>(flag, t, 1 + rep % 7);
      unsigned long long h[3];
      CK(hipMemcpyAsync(h, t, sizeof(h), hipMemcpyDeviceToHost, s));
      CK(hipStreamSynchronize(s));
      if (h[2]) {
        std::printf("flag poll gave up\n");
        return 1;
      }
      if (h[1] >= h[0]) lat.push_back((h[1] - h[0]) * 0.01);  // 100 MHz clock: 10 ns a tick
    }
    if (lat.empty()) {
      std::printf("flag: no ordered sample\n");
      return 1;
    }
    std::sort(lat.begin(), lat.end());
    std::printf("flag_visibility median %.2f us min %.2f us max %.2f us\n", lat[lat.size() / 2],
                lat.front(), lat.back());
    CK(hipFree(flag));
    CK(hipFree(t));
  }
  CK(hipFree(sink));
  return 0;
}
