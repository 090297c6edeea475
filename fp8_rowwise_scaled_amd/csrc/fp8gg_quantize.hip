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
// call moves 3 bytes per element (2 read, 1 written) and is bound by HBM, so the
// per-element arithmetic is kept short:
//   * the quotient x / s is formed from the row's reciprocal r = 1 / s (one IEEE
//     division per row) and two FMA correction steps per element,
//         q = x r;  q += (x - q s) r;  q += (x - q s) r,
//     which is the correctly rounded quotient by Markstein's theorem (r correctly
//     rounded, the first corrected q faithful, each residual x - q s exact).  The
//     residuals are exact as long as nothing underflows, which holds for
//     s >= 2^-64; rows with a smaller scale use the IEEE division itself;
//   * the code comes from the hardware fp8 convert (v_cvt_pk_fp8_f32: OCP e4m3fn,
//     round to nearest even), two values per instruction, on the clamped quotient,
//     with the input's sign bit copied into each code (the convert returns +0 for
//     a zero result, the encoding keeps -0 as 0x80).
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

// Rows whose scale is at least this use the reciprocal-and-correction quotient.
constexpr float kFastScaleMin = 0x1p-64f;

// RN(x / s) from r = RN(1 / s): see the file header.
__device__ __forceinline__ float quotient(float x, float s, float r) {
  float q = x * r;
  q = __builtin_fmaf(__builtin_fmaf(-q, s, x), r, q);
  return __builtin_fmaf(__builtin_fmaf(-q, s, x), r, q);
}

// Eight bf16 values -> eight e4m3fn codes (little-endian bytes in two words).
// FAST: the row's scale admits the reciprocal quotient (else IEEE division).
template <bool FAST>
__device__ __forceinline__ v2i_q quantize8(const v4i_q& v, float s, float r) {
  int w[2] = {0, 0};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float a = FAST ? quotient(bf16_lo(v[j]), s, r) : bf16_lo(v[j]) / s;
    const float b = FAST ? quotient(bf16_hi(v[j]), s, r) : bf16_hi(v[j]) / s;
    // elements 2j and 2j + 1 to bytes 2j and 2j + 1: half j & 1 of word j >> 1
    if (j & 1) w[j >> 1] = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), clamp448(b), w[j >> 1], true);
    else w[j >> 1] = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), clamp448(b), w[j >> 1], false);
  }
  // The convert writes a zero result as +0 (code 0x00); the code keeps the
  // quotient's sign, which is the input's (s > 0): OR each input's sign bit into
  // its byte (a no-op for non-zero codes, which carry it already).
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t lo = (uint32_t)v[2 * h], hi = (uint32_t)v[2 * h + 1];
    const uint32_t sign = ((lo >> 8) & 0x80u) | ((lo >> 16) & 0x8000u) | ((hi << 8) & 0x800000u) | (hi & 0x80000000u);
    w[h] = (int)((uint32_t)w[h] | sign);
  }
  return v2i_q{w[0], w[1]};
}

// At least six waves per SIMD (76 VGPRs, no spills): more rows in flight per CU;
// measured 5% faster than the compiler's own choice (91 VGPRs, five waves).
__global__ void __launch_bounds__(kQThreads) __attribute__((amdgpu_waves_per_eu(6))) quantize_rowwise_kernel(const v4i_q* __restrict__ X,
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
    if (s >= kFastScaleMin) {
      const float r = 1.f / s;
      if (in_regs) {
#pragma unroll
        for (int i = 0; i < kQRegVecs; ++i) {
          const int64_t j = (int64_t)i * kQThreads + tid;
          if (j < nvec) qr[j] = quantize8<true>(held[i], s, r);
        }
      } else {
        for (int64_t j = tid; j < nvec; j += kQThreads) qr[j] = quantize8<true>(xr[j], s, r);
      }
    } else {
      if (in_regs) {
#pragma unroll
        for (int i = 0; i < kQRegVecs; ++i) {
          const int64_t j = (int64_t)i * kQThreads + tid;
          if (j < nvec) qr[j] = quantize8<false>(held[i], s, 0.f);
        }
      } else {
        for (int64_t j = tid; j < nvec; j += kQThreads) qr[j] = quantize8<false>(xr[j], s, 0.f);
      }
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
