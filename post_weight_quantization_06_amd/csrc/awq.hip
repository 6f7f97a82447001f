// Pre-scale hook for composing AAAC with AWQ (AAAC summary §4: AAAC applied to weights that AWQ
// scaled before quantization). Given a positive per-column scale a, the matrix that gets quantized
// is W diag(a) and the importance that matches it is I / a^2: at inference the column k input is
// divided by a_k, so its energy is I_k / a_k^2 and the weighted error of the scaled matrix equals
// the error of the original one.
//
//   W_scaled[r, c] = bf16(W[r, c] * a[c])   the product of a bf16 and an fp32 value has at most 32
//                                           significant bits, exact in fp64; one rounding (ties
//                                           to even) from there
//   I_scaled[c]    = fp32(I[c] / a[c]^2)    a^2 exact in fp64, one fp64 division, then fp32
//
// Elementwise and HBM-bound: 2 B read and 2 B written per weight; a and I stay in cache.
#include "common.h"

namespace aaac {

namespace {

// Round a finite fp64 value to bf16 bits (ties to even), overflowing to infinity past the bf16
// range. In the normal range the rounding works on the fp64 bit pattern at the 8th significant
// bit; below 2^-126 the bf16 quantum is the fixed 2^-133 and adding 1.5 * 2^-81 rounds to it.
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double x) {
  const double ax = fabs(x);
  double r;
  if (ax < 0x1p-126) {
    const double c = 0x1.8p-81;
    r = (ax + c) - c;
  } else {
    uint64_t b = (uint64_t)__double_as_longlong(ax);
    b += 0x00000FFFFFFFFFFFull + ((b >> 45) & 1u);
    b &= ~((1ull << 45) - 1u);
    r = __longlong_as_double((long long)b);
  }
  // r is a bf16 value (exact in fp32) or at least 2^128, which converts to infinity
  const uint32_t bits = __float_as_uint((float)r) >> 16;
  return bits | (__double_as_longlong(x) < 0 ? 0x8000u : 0u);
}

__global__ __launch_bounds__(kBlock) void awq_prescale_kernel(const uint4* __restrict__ W,
                                                              int64_t nvec, int64_t C8,
                                                              const float4* __restrict__ a,
                                                              const float* __restrict__ I,
                                                              int64_t C, uint4* __restrict__ Ws,
                                                              float* __restrict__ Is) {
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  const int64_t first = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  // column vector of element i, advanced by counting (C8 < 2^28)
  const int32_t step = (int32_t)(stride % C8);
  int32_t cv = (int32_t)(first % C8);
  for (int64_t i = first; i < nvec; i += stride) {
    const uint4 v = W[i];
    const float4 a0 = a[2 * cv], a1 = a[2 * cv + 1];
    const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const double lo = (double)__uint_as_float(wv[k] << 16) * (double)av[2 * k];
      const double hi = (double)__uint_as_float(wv[k] & 0xffff0000u) * (double)av[2 * k + 1];
      o[k] = f64_to_bf16_rne(lo) | (f64_to_bf16_rne(hi) << 16);
    }
    Ws[i] = make_uint4(o[0], o[1], o[2], o[3]);
    cv += step;
    if (cv >= C8) cv -= (int32_t)C8;
  }
  if (Is != nullptr) {
    const float* af = reinterpret_cast<const float*>(a);
    for (int64_t k = first; k < C; k += stride) {
      const double ak = (double)af[k];
      Is[k] = (float)((double)I[k] / (ak * ak));
    }
  }
}

}  // namespace

hipError_t launch_awq_prescale(const uint16_t* W, int64_t R, int64_t C, const float* a,
                               const float* I, uint16_t* W_scaled, float* I_scaled,
                               hipStream_t stream) {
  const int64_t nvec = R * C / 8;
  const int64_t want = (nvec + kBlock - 1) / kBlock;
  const int64_t cap = (int64_t)device_cu_count() * 8;
  const int grid = (int)(want < cap ? want : cap);
  hipLaunchKernelGGL(awq_prescale_kernel, dim3(grid), dim3(kBlock), 0, stream,
                     reinterpret_cast<const uint4*>(W), nvec, C / 8,
                     reinterpret_cast<const float4*>(a), I, C, reinterpret_cast<uint4*>(W_scaled),
                     I_scaled);
  return hipGetLastError();
}

}  // namespace aaac
