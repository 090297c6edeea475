// Rowwise fp8 (e4m3fn) quantisation of bf16 activations for gfx950: the step
// that produces the grouped GEMM's XQ and x_scale operands.
//
// Per row (the scheme fixed by MSLK pull request 471's Design notes, scaling-scheme
// paragraph: one scale per row of A, constant along K; the amax choice of the
// scale is this library's reading):
//     s = amax(|x|) / 448 (fp32, IEEE division; 1 for an all-zero row),
//     q = e4m3fn_rne(clamp(x / s, -448, 448))   (fp32 quotient, IEEE division).
//
// One workgroup of 256 threads per row (grid-stride over rows).  A row of up to
// 8192 values is read once into registers (16 bytes = 8 values per load, four
// loads per thread); longer rows are read twice, the second time from L2.  The
// call moves 3 bytes per element (2 read, 1 written) and is bound by HBM.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8gg_internal.h"

namespace fp8gg {

namespace {

typedef int v4i_q __attribute__((ext_vector_type(4)));
typedef int v2i_q __attribute__((ext_vector_type(2)));

constexpr int kQThreads = 256;
constexpr int kQRegVecs = 4;      // 16-byte vectors per thread held across the two passes
constexpr float kE4M3Max = 448.0f;

// e4m3fn code of an fp32 value with |v| <= 448, round to nearest, ties to even.
// Below 2^-6 the format is subnormal with a fixed step of 2^-9, so the code is the
// rounded multiple of that step (8 rounds up into the smallest normal, code 8).
// Above, rounding the fp32 pattern's exponent and top three mantissa bits as one
// integer (ties to even) carries into the exponent by itself; rebasing the
// exponent from bias 127 to bias 7 gives the code.  The sign bit is copied.
__device__ __forceinline__ uint32_t e4m3fn_rne(float v) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t sign = (b >> 24) & 0x80u;
  const uint32_t mag = b & 0x7FFFFFFFu;
  uint32_t code;
  if (mag < 0x3C800000u) {
    code = (uint32_t)__builtin_rintf(__uint_as_float(mag) * 512.0f);
  } else {
    const uint32_t r = (mag + 0x7FFFFu + ((mag >> 20) & 1u)) >> 20;
    code = r - ((127u - 7u) << 3);
  }
  return sign | code;
}

__device__ __forceinline__ float bf16_lo(int w) { return __uint_as_float((uint32_t)w << 16); }
__device__ __forceinline__ float bf16_hi(int w) { return __uint_as_float((uint32_t)w & 0xFFFF0000u); }

__device__ __forceinline__ float amax8(const v4i_q& v, float m) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    m = fmaxf(m, fabsf(bf16_lo(v[j])));
    m = fmaxf(m, fabsf(bf16_hi(v[j])));
  }
  return m;
}

__device__ __forceinline__ float clamp448(float y) {
  // comparisons, not fminf/fmaxf, so that a NaN quotient stays NaN
  return y > kE4M3Max ? kE4M3Max : (y < -kE4M3Max ? -kE4M3Max : y);
}

// Eight bf16 values -> eight e4m3fn codes (little-endian bytes in two words).
__device__ __forceinline__ v2i_q quantize8(const v4i_q& v, float s) {
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t lo = e4m3fn_rne(clamp448(bf16_lo(v[j]) / s));
    const uint32_t hi = e4m3fn_rne(clamp448(bf16_hi(v[j]) / s));
    w[j >> 1] |= (lo | (hi << 8)) << (16 * (j & 1));
  }
  return v2i_q{(int)w[0], (int)w[1]};
}

__global__ void __launch_bounds__(kQThreads) quantize_rowwise_kernel(const v4i_q* __restrict__ X,
                                                                     v2i_q* __restrict__ XQ,
                                                                     float* __restrict__ xs, int64_t rows,
                                                                     int64_t K) {
  __shared__ float wave_max[kQThreads / 64];
  const int tid = threadIdx.x;
  const int64_t nvec = K / 8;
  const bool in_regs = nvec <= (int64_t)kQThreads * kQRegVecs;
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const v4i_q* xr = X + row * nvec;
    v4i_q held[kQRegVecs];
    float m = 0.f;
    if (in_regs) {
#pragma unroll
      for (int i = 0; i < kQRegVecs; ++i) {
        const int64_t j = (int64_t)i * kQThreads + tid;
        held[i] = j < nvec ? xr[j] : v4i_q{0, 0, 0, 0};
        m = amax8(held[i], m);
      }
    } else {
      for (int64_t j = tid; j < nvec; j += kQThreads) m = amax8(xr[j], m);
    }
    // workgroup max: within each wave, then across the four waves through LDS
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    if ((tid & 63) == 0) wave_max[tid >> 6] = m;
    __syncthreads();
    float amax = wave_max[0];
#pragma unroll
    for (int w = 1; w < kQThreads / 64; ++w) amax = fmaxf(amax, wave_max[w]);
    __syncthreads();   // wave_max is rewritten by the next row
    const float s = amax > 0.f ? amax / kE4M3Max : 1.f;
    v2i_q* qr = XQ + row * nvec;
    if (in_regs) {
#pragma unroll
      for (int i = 0; i < kQRegVecs; ++i) {
        const int64_t j = (int64_t)i * kQThreads + tid;
        if (j < nvec) qr[j] = quantize8(held[i], s);
      }
    } else {
      for (int64_t j = tid; j < nvec; j += kQThreads) qr[j] = quantize8(xr[j], s);
    }
    if (tid == 0) xs[row] = s;
  }
}

}  // namespace

hipError_t launch_quantize_rowwise(const uint16_t* X, uint8_t* XQ, float* x_scale, int64_t rows, int64_t K,
                                   hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int64_t grid = rows < 8192 ? rows : 8192;
  hipLaunchKernelGGL(quantize_rowwise_kernel, dim3((uint32_t)grid), dim3(kQThreads), 0, stream,
                     reinterpret_cast<const v4i_q*>(X), reinterpret_cast<v2i_q*>(XQ), x_scale, rows, K);
  return hipGetLastError();
}

}  // namespace fp8gg
