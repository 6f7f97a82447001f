// Refine step (AAAC summary §2 mechanism 4): activation-weighted k-means update of both tables.
//
// For every cell (table c, entry j) the kernel sums num = sum I_k s w_k and den = sum I_k s^2 over
// the weights whose selection group chose c and whose code is j; the new entry is num / den (the
// minimizer of sum I (w - s t)^2), or the old entry if the cell is empty.
//
// Accumulation: every thread owns a private column of 64 fp32 bins in LDS (32 cells x {num, den},
// laid out [bin][thread] so a wave's adds hit 64 different banks) and adds at most 64 terms into a
// bin before it moves the bin into fp64 registers. Workgroups then reduce their 256 threads in a
// fixed order and write one fp64 partial per (cell, workgroup); a second kernel adds the partials of
// each cell in a fixed order and divides. No float atomics touch global memory and every order is
// fixed, so results are bitwise reproducible.
#include "common.h"

namespace aaac {

namespace {

constexpr int kCells = 32;   // 2 tables x 16 entries
constexpr int kVals = 64;    // num and den per cell

struct RefineShared {
  float num[kCells][kBlock];
  float den[kCells][kBlock];
};

// Fixed-order reduction of acc[64] over the 256 threads of the block; thread t < 32 of half h
// returns value 32 h + t through `out`. Uses the (zero) bins as scratch and zeroes them again.
__device__ void block_reduce_acc(RefineShared& sh, double (&acc)[kVals], double* out_lo,
                                 double* out_hi) {
  const int tid = threadIdx.x;
  double* scratch = reinterpret_cast<double*>(&sh);   // 64 KB = 32 x 256 doubles
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    __syncthreads();
#pragma unroll
    for (int v = 0; v < 32; ++v) scratch[v * kBlock + tid] = acc[32 * h + v];
    __syncthreads();
    const int v = tid & 31, part = tid >> 5;
    double s = 0.0;
    for (int i = 0; i < 32; ++i) {
      const int col = part * 32 + ((i + v) & 31);
      s += scratch[v * kBlock + col];
    }
    __syncthreads();
    scratch[v * 8 + part] = s;
    __syncthreads();
    if (tid < 32) {
      double t = 0.0;
      for (int p = 0; p < 8; ++p) t += scratch[tid * 8 + p];
      if (h == 0) *out_lo = t; else *out_hi = t;
    }
  }
  __syncthreads();
  for (int k = 0; k < kCells; ++k) {
    sh.num[k][tid] = 0.0f;
    sh.den[k][tid] = 0.0f;
  }
  __syncthreads();
}

__device__ __forceinline__ void flush_bins(RefineShared& sh, double (&acc)[kVals]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int k = 0; k < kCells; ++k) {
    acc[k] += (double)sh.num[k][tid];
    acc[kCells + k] += (double)sh.den[k][tid];
    sh.num[k][tid] = 0.0f;
    sh.den[k][tid] = 0.0f;
  }
}

__device__ __forceinline__ void write_partials(const RefineBatch& b, int job, double lo,
                                               double hi) {
  // thread t < 32 holds values t (num of cell t) and 32 + t (den of cell t)
  const int tid = threadIdx.x;
  if (tid < 32) {
    double* base = b.partials + (size_t)job * kVals * b.nblocks;
    base[(size_t)tid * b.nblocks + blockIdx.x] = lo;
    base[(size_t)(32 + tid) * b.nblocks + blockIdx.x] = hi;
  }
}

}  // namespace

__global__ __launch_bounds__(kBlock, 2) void refine_accum_kernel(RefineBatch b) {
  __shared__ RefineShared sh;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int g8 = b.g / kPerLane, S = b.S;
  for (int k = 0; k < kCells; ++k) {
    sh.num[k][tid] = 0.0f;
    sh.den[k][tid] = 0.0f;
  }
  double acc[kVals];
#pragma unroll
  for (int k = 0; k < kVals; ++k) acc[k] = 0.0;
  int cur = -1;
  uint32_t touched = 0;
  for (int64_t task = blockIdx.x; task < b.total_tasks; task += gridDim.x) {
    int j = 0;
    while (j + 1 < b.njobs && task >= b.job[j + 1].geom.task_begin) ++j;
    if (j != cur) {
      if (cur >= 0) {
        double lo = 0.0, hi = 0.0;
        block_reduce_acc(sh, acc, &lo, &hi);
        write_partials(b, cur, lo, hi);
#pragma unroll
        for (int k = 0; k < kVals; ++k) acc[k] = 0.0;
      }
      cur = j;
      touched |= 1u << j;
    }
    const RefineJob& jb = b.job[j];
    const int64_t local = task - jb.geom.task_begin;
    const int64_t rb = local / jb.geom.nslab;
    const int slab = (int)(local - rb * jb.geom.nslab);
    const int c0 = slab * kSlab + lane * kPerLane;
    const bool active = c0 < jb.geom.C;
    float Ik[8];
    if (active) {
      const float4 i0 = *reinterpret_cast<const float4*>(jb.I + c0);
      const float4 i1 = *reinterpret_cast<const float4*>(jb.I + c0 + 4);
      Ik[0] = i0.x; Ik[1] = i0.y; Ik[2] = i0.z; Ik[3] = i0.w;
      Ik[4] = i1.x; Ik[5] = i1.y; Ik[6] = i1.z; Ik[7] = i1.w;
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) Ik[k] = 0.0f;
    }
    for (int i = 0; i < kRowsPerWave; ++i) {
      const int64_t r = rb * kRowsPerTask + wave + (int64_t)kWavesPerBlock * i;
      if (r >= jb.geom.R) break;
      const int64_t base = r * (int64_t)jb.geom.C + c0;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      uint32_t cw = 0, sb = 0;
      if (active) {
        v = *reinterpret_cast<const uint4*>(jb.W + base);
        cw = jb.codes[base >> 3];
        sb = jb.sel[base / S];
      }
      const uint32_t amax = block_max_u32(lane_absmax_bits(v), g8);
      const float s = __uint_as_float(amax << 16);
      if (active) {
        float w[8];
        unpack8(v, w);
        const int cbase = sb ? 16 : 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int cell = cbase + ((cw >> (4 * k)) & 15u);
          const float t = Ik[k] * s;
          atomicAdd(&sh.num[cell][tid], t * w[k]);
          atomicAdd(&sh.den[cell][tid], t * s);
        }
      }
    }
    flush_bins(sh, acc);
  }
  if (cur >= 0) {
    double lo = 0.0, hi = 0.0;
    block_reduce_acc(sh, acc, &lo, &hi);
    write_partials(b, cur, lo, hi);
  }
  for (int j = 0; j < b.njobs; ++j)
    if (!(touched & (1u << j))) write_partials(b, j, 0.0, 0.0);
}

// Round a finite fp64 value to bf16 (ties to even) directly, without an intermediate fp32
// rounding: the quantum of x's binade (8 significant bits; below 2^-126 the fixed subnormal quantum
// 2^-133) divides x exactly, rint rounds half to even, and the product is exact.
__device__ __forceinline__ float f64_to_bf16_value(double x) {
  if (x == 0.0 || !isfinite(x)) return (float)x;
  const double ax = fabs(x);
  const int e = ax < 0x1p-126 ? -126 : ilogb(ax);
  const double q = ldexp(1.0, e - 7);
  double r = rint(ax / q) * q;
  if (r >= 0x1p128) r = __builtin_inf();
  return (float)copysign(r, x);
}

__global__ __launch_bounds__(kBlock) void refine_finalize_kernel(RefineBatch b) {
  const int j = blockIdx.x / kCells, cell = blockIdx.x % kCells;
  const int c = cell >> 4, idx = cell & 15;
  if (idx >= b.n) return;
  const int tid = threadIdx.x;
  const double* pn = b.partials + ((size_t)j * kVals + cell) * b.nblocks;
  const double* pd = b.partials + ((size_t)j * kVals + kCells + cell) * b.nblocks;
  double sn = 0.0, sd = 0.0;
  for (int i = tid; i < b.nblocks; i += kBlock) {
    sn += pn[i];
    sd += pd[i];
  }
  __shared__ double rn[kBlock], rd[kBlock];
  rn[tid] = sn;
  rd[tid] = sd;
  __syncthreads();
  for (int w = kBlock / 2; w > 0; w >>= 1) {
    if (tid < w) {
      rn[tid] += rn[tid + w];
      rd[tid] += rd[tid + w];
    }
    __syncthreads();
  }
  if (tid == 0) {
    const RefineJob& jb = b.job[j];
    const float old = jb.tables_in[c * b.n + idx];
    const double val = rd[0] > 0.0 ? rn[0] / rd[0] : (double)old;
    jb.tables_out[c * b.n + idx] = (b.flags & 1) ? f64_to_bf16_value(val) : (float)val;
  }
}

int refine_grid(int64_t total_tasks) {
  const int64_t want = (int64_t)device_cu_count() * 2;
  return (int)(total_tasks < want ? total_tasks : want);
}

hipError_t launch_refine(RefineBatch& b, hipStream_t stream) {
  if (b.nblocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(refine_accum_kernel, dim3(b.nblocks), dim3(kBlock), 0, stream, b);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(refine_finalize_kernel, dim3(b.njobs * kCells), dim3(kBlock), 0, stream, b);
  return hipGetLastError();
}

}  // namespace aaac
