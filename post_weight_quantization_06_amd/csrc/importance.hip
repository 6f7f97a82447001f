// Importance (AAAC summary §2 mechanism 2): I_k = sum_t X[t, k]^2 over the calibration tokens.
//
// Pass 1: the token axis is cut into `nsplit` contiguous ranges; a thread owns VEC consecutive
// columns of one range and sums the exact fp64 squares in token order (coalesced: a wave reads
// 64 * VEC consecutive floats of a row). Pass 2 adds the range sums to the running fp64
// accumulator and writes the fp32 copy. Fixed order, no atomics.
#include "common.h"

namespace aaac {

template <int VEC>
__global__ __launch_bounds__(kBlock) void importance_partial_kernel(const float* __restrict__ X,
                                                                    int64_t T, int64_t K,
                                                                    int64_t ldx, int64_t chunk,
                                                                    double* __restrict__ partials) {
  const int64_t col = ((int64_t)blockIdx.x * kBlock + threadIdx.x) * VEC;
  if (col >= K) return;
  const int64_t t0 = (int64_t)blockIdx.y * chunk;
  const int64_t t1 = t0 + chunk < T ? t0 + chunk : T;
  double acc[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) acc[v] = 0.0;
  const float* p = X + t0 * ldx + col;
  int64_t t = t0;
  if (VEC == 4) {
    for (; t + 4 <= t1; t += 4, p += 4 * ldx) {
      float4 x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = *reinterpret_cast<const float4*>(p + u * ldx);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        acc[0] += (double)x[u].x * (double)x[u].x;
        acc[1 % VEC] += (double)x[u].y * (double)x[u].y;
        acc[2 % VEC] += (double)x[u].z * (double)x[u].z;
        acc[3 % VEC] += (double)x[u].w * (double)x[u].w;
      }
    }
    for (; t < t1; ++t, p += ldx) {
      const float4 x = *reinterpret_cast<const float4*>(p);
      acc[0] += (double)x.x * (double)x.x;
      acc[1 % VEC] += (double)x.y * (double)x.y;
      acc[2 % VEC] += (double)x.z * (double)x.z;
      acc[3 % VEC] += (double)x.w * (double)x.w;
    }
  } else {
    for (; t < t1; ++t, p += ldx) {
#pragma unroll
      for (int v = 0; v < VEC; ++v) acc[v] += (double)p[v] * (double)p[v];
    }
  }
  double* out = partials + (int64_t)blockIdx.y * K + col;
#pragma unroll
  for (int v = 0; v < VEC; ++v) out[v] = acc[v];
}

// Pass 2: a workgroup takes 16 columns; thread group q (16 of them) adds the range sums q, q + 16,
// q + 32, ... of its column in that order, then group 0 adds the 16 group sums in group order to
// the running accumulator. Every order is fixed.
constexpr int kFinCols = 16;
constexpr int kFinGroups = kBlock / kFinCols;

__global__ __launch_bounds__(kBlock) void importance_finalize_kernel(const double* __restrict__ partials,
                                                                     int nsplit, int64_t K,
                                                                     double* I_acc, float* I_out) {
  __shared__ double part[kFinGroups][kFinCols];
  const int c = threadIdx.x % kFinCols, q = threadIdx.x / kFinCols;
  const int64_t k = (int64_t)blockIdx.x * kFinCols + c;
  double s = 0.0;
  if (k < K) {
#pragma unroll 8
    for (int i = q; i < nsplit; i += kFinGroups) s += partials[(int64_t)i * K + k];
  }
  part[q][c] = s;
  __syncthreads();
  if (q == 0 && k < K) {
    double sum = 0.0;
#pragma unroll
    for (int i = 0; i < kFinGroups; ++i) sum += part[i][c];
    const double tot = I_acc[k] + sum;
    I_acc[k] = tot;
    if (I_out) I_out[k] = (float)tot;
  }
}

int importance_splits(int64_t T, int64_t K) {
  if (T <= 0) return 0;
  const int64_t colblocks = (K + kBlock * 4 - 1) / (kBlock * 4);
  int64_t want = (2048 + colblocks - 1) / colblocks;
  const int64_t most = (T + 63) / 64;      // at least 64 tokens per range
  if (want > most) want = most;
  if (want > 1024) want = 1024;
  if (want < 1) want = 1;
  return (int)want;
}

hipError_t launch_importance(const float* X, int64_t T, int64_t K, int64_t ldx, double* I_acc,
                             float* I_out, double* partials, int nsplit, hipStream_t stream) {
  if (nsplit > 0) {
    const int64_t chunk = (T + nsplit - 1) / nsplit;
    const bool vec = (K % 4 == 0) && (ldx % 4 == 0) && ((uintptr_t)X % 16 == 0);
    if (vec) {
      const dim3 grid((unsigned)((K / 4 + kBlock - 1) / kBlock), (unsigned)nsplit);
      hipLaunchKernelGGL(importance_partial_kernel<4>, grid, dim3(kBlock), 0, stream, X, T, K, ldx,
                         chunk, partials);
    } else {
      const dim3 grid((unsigned)((K + kBlock - 1) / kBlock), (unsigned)nsplit);
      hipLaunchKernelGGL(importance_partial_kernel<1>, grid, dim3(kBlock), 0, stream, X, T, K, ldx,
                         chunk, partials);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(importance_finalize_kernel, dim3((unsigned)((K + kFinCols - 1) / kFinCols)),
                     dim3(kBlock), 0, stream, partials, nsplit, K, I_acc, I_out);
  return hipGetLastError();
}

}  // namespace aaac
