// Measured device peaks for gfx950: a matrix-core-only kernel (fp8 and bf16)
// and HBM read / copy kernels, each timed with HIP events.  See
// include/dsa_peak.h for the contract.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsa_peak.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int MF_NT = 256;        // threads per workgroup
constexpr int MF_WG_PER_CU = 4;   // 16 waves per CU, 4 per SIMD
constexpr int MF_CHAINS = 4;      // independent accumulators per wave
constexpr int MF_ITERS = 4096;    // loop trips per wave

// Every wave issues MF_ITERS * MF_CHAINS independent MFMAs.  The operands
// depend on the thread id, and the results are stored only when `flag` is
// set (never, at run time), so nothing is folded away.  Wave 0 of
// workgroup 0 records the shader clock and the constant 100 MHz clock
// around its loop.
template <bool FP8>
__global__ void __launch_bounds__(MF_NT) mfma_peak_kernel(int flag, float* sink, long long* clk) {
  const int tid = threadIdx.x;
  v16f acc[MF_CHAINS];
#pragma unroll
  for (int c = 0; c < MF_CHAINS; ++c) acc[c] = v16f{};
  const long long t0 = __builtin_amdgcn_s_memtime();
  const long long r0 = __builtin_amdgcn_s_memrealtime();
  if constexpr (FP8) {
    const v8i a = v8i{tid, tid + 1, tid + 2, tid + 3, tid + 4, tid + 5, tid + 6, tid + 7} & 0x37373737;
    const v8i b = a ^ 0x01010101;
    for (int i = 0; i < MF_ITERS; ++i) {
#pragma unroll
      for (int c = 0; c < MF_CHAINS; ++c)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 0, 0, 0, 127, 0, 127);
    }
  } else {
    const v4i ai = v4i{tid, tid + 1, tid + 2, tid + 3} & 0x3F003F00;
    const v8bf a = __builtin_bit_cast(v8bf, ai);
    const v8bf b = __builtin_bit_cast(v8bf, ai ^ 0x00100010);
    for (int i = 0; i < MF_ITERS; ++i) {
#pragma unroll
      for (int c = 0; c < MF_CHAINS; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
  }
  const long long t1 = __builtin_amdgcn_s_memtime();
  const long long r1 = __builtin_amdgcn_s_memrealtime();
  if (blockIdx.x == 0 && tid == 0) {
    clk[0] = t1 - t0;
    clk[1] = r1 - r0;
  }
  if (flag) {
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < MF_CHAINS; ++c)
#pragma unroll
      for (int j = 0; j < 16; ++j) s += acc[c][j];
    sink[blockIdx.x * MF_NT + tid] = s;
  }
}

constexpr int RD_NT = 256;
constexpr int RD_UNROLL = 8;      // 16-byte loads in flight per thread

// Grid-stride read of n16 16-byte vectors, RD_UNROLL loads issued before any
// is used; the xor of everything read is stored only when it equals a value
// no input produces by chance and `flag` is set.
__global__ void __launch_bounds__(RD_NT) hbm_read_kernel(const v4i* __restrict__ p, size_t n16, int flag,
                                                         int* sink) {
  const size_t stride = (size_t)gridDim.x * RD_NT;
  size_t i = (size_t)blockIdx.x * RD_NT + threadIdx.x;
  v4i acc = v4i{0, 0, 0, 0};
  for (; i + (RD_UNROLL - 1) * stride < n16; i += RD_UNROLL * stride) {
    v4i v[RD_UNROLL];
#pragma unroll
    for (int u = 0; u < RD_UNROLL; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < RD_UNROLL; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= p[i];
  if (flag && (acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == flag) sink[threadIdx.x] = acc[0];
}

__global__ void __launch_bounds__(RD_NT) hbm_copy_kernel(const v4i* __restrict__ src, v4i* __restrict__ dst,
                                                         size_t n16) {
  const size_t stride = (size_t)gridDim.x * RD_NT;
  size_t i = (size_t)blockIdx.x * RD_NT + threadIdx.x;
  for (; i + (RD_UNROLL - 1) * stride < n16; i += RD_UNROLL * stride) {
    v4i v[RD_UNROLL];
#pragma unroll
    for (int u = 0; u < RD_UNROLL; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < RD_UNROLL; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

int device_cus(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
  return (int)e;
}

// Times `launch` over `iters` launches after one warm-up; *ms = mean.
template <class F>
int time_launches(F launch, int iters, hipStream_t s, double* ms) {
  if (iters < 1) return (int)hipErrorInvalidValue;
  hipEvent_t a, b;
  hipError_t e = hipEventCreate(&a);
  if (e != hipSuccess) return (int)e;
  e = hipEventCreate(&b);
  if (e != hipSuccess) {
    (void)hipEventDestroy(a);
    return (int)e;
  }
  launch();
  e = hipGetLastError();
  if (e == hipSuccess) e = hipEventRecord(a, s);
  for (int i = 0; e == hipSuccess && i < iters; ++i) {
    launch();
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipEventRecord(b, s);
  if (e == hipSuccess) e = hipEventSynchronize(b);
  float el = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&el, a, b);
  (void)hipEventDestroy(a);
  (void)hipEventDestroy(b);
  *ms = (double)el / iters;
  return (int)e;
}

template <bool FP8>
int mfma_peak(int iters, double* tflops, double* clock_mhz, hipStream_t s) {
  if (!tflops) return (int)hipErrorInvalidValue;
  int cus = 0;
  int e = device_cus(&cus);
  if (e) return e;
  const int grid = cus * MF_WG_PER_CU;
  long long* clk = nullptr;
  hipError_t he = hipMalloc(&clk, 2 * sizeof(long long));
  if (he != hipSuccess) return (int)he;
  double ms = 0.0;
  e = time_launches([&]() {
    hipLaunchKernelGGL(mfma_peak_kernel<FP8>, dim3(grid), dim3(MF_NT), 0, s, 0, nullptr, clk);
  }, iters, s, &ms);
  long long hc[2] = {0, 0};
  if (!e) e = (int)hipMemcpy(hc, clk, sizeof(hc), hipMemcpyDeviceToHost);
  (void)hipFree(clk);
  if (e) return e;
  const double flop_per_mfma = FP8 ? 2.0 * 32 * 32 * 64 : 2.0 * 32 * 32 * 16;
  const double mfmas = (double)grid * (MF_NT / 64) * MF_ITERS * MF_CHAINS;
  *tflops = mfmas * flop_per_mfma / (ms * 1e-3) / 1e12;
  if (clock_mhz) *clock_mhz = hc[1] > 0 ? 100.0 * (double)hc[0] / (double)hc[1] : 0.0;
  return 0;
}

}  // namespace

extern "C" {

int dsa_peak_mfma_fp8(int iters, double* tflops, double* clock_mhz, void* stream) {
  return mfma_peak<true>(iters, tflops, clock_mhz, static_cast<hipStream_t>(stream));
}

int dsa_peak_mfma_bf16(int iters, double* tflops, double* clock_mhz, void* stream) {
  return mfma_peak<false>(iters, tflops, clock_mhz, static_cast<hipStream_t>(stream));
}

int dsa_peak_hbm_read(const void* buf, size_t bytes, int iters, double* gbps, void* stream) {
  if (!buf || !gbps || bytes < (1u << 20) || bytes % 16 || (reinterpret_cast<uintptr_t>(buf) & 15u))
    return (int)hipErrorInvalidValue;
  int cus = 0;
  int e = device_cus(&cus);
  if (e) return e;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int grid = cus * 32;
  double ms = 0.0;
  e = time_launches([&]() {
    hipLaunchKernelGGL(hbm_read_kernel, dim3(grid), dim3(RD_NT), 0, s, static_cast<const v4i*>(buf), bytes / 16, 0,
                       nullptr);
  }, iters, s, &ms);
  if (e) return e;
  *gbps = (double)bytes / (ms * 1e-3) / 1e9;
  return 0;
}

int dsa_peak_hbm_copy(const void* src, void* dst, size_t bytes, int iters, double* gbps, void* stream) {
  if (!src || !dst || !gbps || bytes < (1u << 20) || bytes % 16 ||
      ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15u))
    return (int)hipErrorInvalidValue;
  int cus = 0;
  int e = device_cus(&cus);
  if (e) return e;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int grid = cus * 32;
  double ms = 0.0;
  e = time_launches([&]() {
    hipLaunchKernelGGL(hbm_copy_kernel, dim3(grid), dim3(RD_NT), 0, s, static_cast<const v4i*>(src),
                       static_cast<v4i*>(dst), bytes / 16);
  }, iters, s, &ms);
  if (e) return e;
  *gbps = 2.0 * (double)bytes / (ms * 1e-3) / 1e9;
  return 0;
}

}  // extern "C"
