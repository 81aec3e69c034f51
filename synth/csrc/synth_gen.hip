// Device implementation of the seeded input generator (the host version is
// synth/gen.py; both produce the same bytes).
//
// Element i of stream (seed, stream) is the i-th output of SplitMix64
// (Steele, Lea and Flood, OOPSLA 2014) started at `base` = mix64(seed<<32 |
// stream), computed on the host.  A normal draw is table[h >> 48] (65536
// equiprobable quantile levels, table supplied by the host).  Only integer
// operations, table lookups and IEEE-rounded float32 multiply / add / divide
// follow, and the library is built with -ffp-contract=off so that no multiply
// and add are fused into an fma.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ float normal_at(uint64_t base, uint64_t i, const float* table) {
  const uint64_t h = mix64(base + (i + 1ull) * 0x9E3779B97F4A7C15ull);
  return table[h >> 48];
}

__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 31) << 7;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a >= 0x3C800000u) {
    const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    const int e = (int)(r >> 23) - 127;
    const uint32_t m = (r >> 20) & 7u;
    if (e > 8 || (e == 8 && m == 7u)) code = 0x7Eu;
    else code = ((uint32_t)(e + 7) << 3) | m;
  } else {
    code = (uint32_t)__builtin_rintf(__fmul_rn(__uint_as_float(a), 512.0f));
  }
  return code | sign;
}

__device__ __forceinline__ uint16_t bf16_code(float x) {
  const uint32_t u = __float_as_uint(x);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// out[r, c] for rows r of a [*, ncols] tensor whose row index is row0 + r:
//   X = N(base_0);  for l in 1..layers: X = rho*X + sigma*N(base_l)
//   then X = X / div (div != 0), then row r times mult[r] (mult may be null).
__global__ void gen_rows_kernel(const uint64_t* bases, int layers, long long row0, int nrows, int ncols,
                                const float* table, float rho, float sigma, float div, const float* mult,
                                float* out) {
  const long long n = (long long)nrows * ncols;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (long long)gridDim.x * blockDim.x) {
    const long long r = e / ncols;
    const uint64_t i = (uint64_t)((row0 + r) * ncols + (e - r * ncols));
    float x = normal_at(bases[0], i, table);
    for (int l = 1; l <= layers; ++l) x = __fadd_rn(__fmul_rn(rho, x), __fmul_rn(sigma, normal_at(bases[l], i, table)));
    if (div != 0.0f) x = __fdiv_rn(x, div);
    if (mult) x = __fmul_rn(x, mult[r]);
    out[e] = x;
  }
}

// per-row e4m3: scale = amax / 448 (1 if amax == 0), code = e4m3(x / scale)
__global__ void quant_rows_kernel(const float* X, int nrows, int ncols, uint8_t* codes, float* scales) {
  __shared__ float red[32];
  const int r = blockIdx.x;
  if (r >= nrows) return;
  const float* x = X + (size_t)r * ncols;
  float amax = 0.f;
  for (int c = threadIdx.x; c < ncols; c += blockDim.x) amax = fmaxf(amax, fabsf(x[c]));
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = 0.f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) amax = fmaxf(amax, red[w]);
  const float scale = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
  for (int c = threadIdx.x; c < ncols; c += blockDim.x)
    codes[(size_t)r * ncols + c] = (uint8_t)e4m3_code(__fdiv_rn(x[c], scale));
  if (threadIdx.x == 0) scales[r] = scale;
}

__global__ void bf16_kernel(const float* X, long long n, uint16_t* out) {
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (long long)gridDim.x * blockDim.x)
    out[e] = bf16_code(X[e]);
}

}  // namespace

extern "C" {

int synth_gen_rows(const uint64_t* bases_dev, int layers, long long row0, int nrows, int ncols, const float* table,
                   float rho, float sigma, float div, const float* mult, float* out, void* stream) {
  const long long n = (long long)nrows * ncols;
  long long blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(gen_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, bases_dev, layers,
                     row0, nrows, ncols, table, rho, sigma, div, mult, out);
  return (int)hipGetLastError();
}

int synth_quant_rows_e4m3(const float* X, int nrows, int ncols, uint8_t* codes, float* scales, void* stream) {
  if (nrows < 1) return 0;
  hipLaunchKernelGGL(quant_rows_kernel, dim3(nrows), dim3(256), 0, (hipStream_t)stream, X, nrows, ncols, codes,
                     scales);
  return (int)hipGetLastError();
}

int synth_bf16(const float* X, long long n, uint16_t* out, void* stream) {
  long long blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, X, n, out);
  return (int)hipGetLastError();
}

}  // extern "C"
