// Refine step (AAAC summary §2 mechanism 4): activation-weighted k-means update of both tables.
//
// For every cell (table c, entry j) the kernel sums num = sum I_k s w_k and den = sum I_k s^2 over
// the weights whose selection group chose c and whose code is j; the new entry is num / den (the
// minimizer of sum I (w - s t)^2), or the old entry if the cell is empty.
//
// Accumulation: each term is exact in fp64 (s w and s^2 have at most 16 significant bits, times
// the 24-bit I), and every thread adds its terms into a private column of 64 fp64 bins in LDS
// (32 cells x {num, den}, laid out [bin][thread]) with ds_add_f64. When a workgroup leaves a matrix
// it reduces its 256 columns in a fixed order and writes one fp64 partial per (bin, workgroup); the
// last workgroup to finish that matrix (an integer ticket) adds the partials in workgroup order and
// divides. Every order is fixed, so results are bitwise reproducible.
//
// The bins take 128 KB, one workgroup per CU; to keep enough bytes in flight each wave loads the
// rows of its next task before it accumulates the current one.
#include "common.h"

namespace aaac {

namespace {

constexpr int kCells = 32;   // 2 tables x 16 entries
constexpr int kVals = 64;    // num (bins 0-31) and den (bins 32-63)

struct RefineShared {
  double bins[kVals][kBlock];
};

struct TaskRows {
  uint4 v[kRowsPerWave];
  uint32_t cw[kRowsPerWave];
  uint32_t sb[kRowsPerWave];
  float I[kPerLane];
  int64_t r0;
  int job;
  int c0;
  bool active;
};

__device__ __forceinline__ void load_task(const RefineBatch& b, int64_t task, int log2S,
                                          TaskRows& t) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  int j = 0;
  while (j + 1 < b.njobs && task >= b.job[j + 1].geom.task_begin) ++j;
  const RefineJob& jb = b.job[j];
  const int64_t local = task - jb.geom.task_begin;
  const int64_t rb = local / jb.geom.nslab;
  const int slab = (int)(local - rb * jb.geom.nslab);
  t.job = j;
  t.c0 = slab * kSlab + lane * kPerLane;
  t.active = t.c0 < jb.geom.C;
  t.r0 = rb * kRowsPerTask + wave;
  const int64_t R = jb.geom.R, C = jb.geom.C;
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    const int64_t r = t.r0 + (int64_t)kWavesPerBlock * i;
    t.v[i] = make_uint4(0u, 0u, 0u, 0u);
    t.cw[i] = 0;
    t.sb[i] = 0;
    if (t.active && r < R) {
      const int64_t base = r * C + t.c0;
      t.v[i] = *reinterpret_cast<const uint4*>(jb.W + base);
      t.cw[i] = jb.codes[base >> 3];
      t.sb[i] = jb.sel[base >> log2S];
    }
  }
  if (t.active) {
    const float4 i0 = *reinterpret_cast<const float4*>(jb.I + t.c0);
    const float4 i1 = *reinterpret_cast<const float4*>(jb.I + t.c0 + 4);
    t.I[0] = i0.x; t.I[1] = i0.y; t.I[2] = i0.z; t.I[3] = i0.w;
    t.I[4] = i1.x; t.I[5] = i1.y; t.I[6] = i1.z; t.I[7] = i1.w;
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) t.I[k] = 0.0f;
  }
}

__device__ __forceinline__ void accumulate_task(const RefineBatch& b, const TaskRows& t, int g8,
                                                RefineShared& sh) {
  const int tid = threadIdx.x;
  const int64_t R = b.job[t.job].geom.R;
  double Id[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) Id[k] = (double)t.I[k];
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    const int64_t r = t.r0 + (int64_t)kWavesPerBlock * i;
    if (r >= R) continue;
    const uint32_t amax = block_max_u32(lane_absmax_bits(t.v[i]), g8);
    if (!t.active) continue;
    const float s = __uint_as_float(amax << 16);
    const double s2 = (double)(s * s);          // exact: s has 8 significant bits
    float w[8];
    unpack8(t.v[i], w);
    const int cbase = t.sb[i] ? 16 : 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int cell = cbase + ((t.cw[i] >> (4 * k)) & 15u);
      atomicAdd(&sh.bins[cell][tid], Id[k] * (double)(s * w[k]));   // s w exact in fp32
      atomicAdd(&sh.bins[kCells + cell][tid], Id[k] * s2);
    }
  }
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

// Publish this workgroup's partial of job j (and zero the bins); the last workgroup of the job adds
// all partials and writes the tables.
__device__ void finish_job(const RefineBatch& b, int j, RefineShared& sh) {
  const int tid = threadIdx.x;
  const RefineJob& jb = b.job[j];
  __shared__ double part4[4][kVals];
  __shared__ uint32_t ticket;
  __syncthreads();
  {
    // value v = tid & 63 over the 64 columns of quarter q = tid >> 6, in a fixed (rotated) order
    const int v = tid & 63, q = tid >> 6;
    double s = 0.0;
    for (int i = 0; i < 64; ++i) s += sh.bins[v][q * 64 + ((i + v) & 63)];
    part4[q][v] = s;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kVals; ++k) sh.bins[k][tid] = 0.0;
  double* part = b.partials + (size_t)j * kVals * b.slots;
  const int slot = (int)blockIdx.x - jb.wg_lo;
  if (tid < kVals) {
    const double tot = ((part4[0][tid] + part4[1][tid]) + part4[2][tid]) + part4[3][tid];
    part[(size_t)tid * b.slots + slot] = tot;
    __threadfence();
  }
  __syncthreads();
  if (tid == 0) ticket = atomicAdd(b.counters + j, 1u);
  __syncthreads();
  if (ticket != (uint32_t)(jb.wg_count - 1)) return;
  // last workgroup of this job: every partial is visible after the fence
  __threadfence();
  {
    const int v = tid & 63, q = tid >> 6;
    const int cnt = jb.wg_count;
    const int s0 = (q * cnt) / 4, s1 = ((q + 1) * cnt) / 4;
    double s = 0.0;
    for (int i = s0; i < s1; ++i) s += part[(size_t)v * b.slots + i];
    part4[q][v] = s;
  }
  __syncthreads();
  if (tid < kCells) {
    const int c = tid >> 4, idx = tid & 15;
    const double nsum = ((part4[0][tid] + part4[1][tid]) + part4[2][tid]) + part4[3][tid];
    const double dsum = ((part4[0][kCells + tid] + part4[1][kCells + tid]) + part4[2][kCells + tid]) +
                        part4[3][kCells + tid];
    if (idx < b.n) {
      const float old = jb.tables_in[c * b.n + idx];
      const double val = dsum > 0.0 ? nsum / dsum : (double)old;
      jb.tables_out[c * b.n + idx] = (b.flags & 1) ? f64_to_bf16_value(val) : (float)val;
    }
  }
  if (tid == 0) b.counters[j] = 0u;
  __syncthreads();
}

}  // namespace

__global__ __launch_bounds__(kBlock, 1) void refine_kernel(RefineBatch b) {
  __shared__ RefineShared sh;
  const int tid = threadIdx.x;
  const int g8 = b.g / kPerLane;
  const int log2S = 31 - __builtin_clz((unsigned)b.S);
#pragma unroll
  for (int k = 0; k < kVals; ++k) sh.bins[k][tid] = 0.0;
  const int64_t t_begin = task_lo(blockIdx.x, b.total_tasks, gridDim.x);
  const int64_t t_end = task_lo(blockIdx.x + 1, b.total_tasks, gridDim.x);
  // two statically named buffers: the rows of task t + 1 load while task t accumulates
  TaskRows A, B;
  int cur = -1;
  if (t_begin < t_end) load_task(b, t_begin, log2S, A);
  for (int64_t task = t_begin; task < t_end; task += 2) {
    if (task + 1 < t_end) load_task(b, task + 1, log2S, B);
    if (A.job != cur) {
      if (cur >= 0) finish_job(b, cur, sh);
      cur = A.job;
    }
    accumulate_task(b, A, g8, sh);
    if (task + 1 >= t_end) break;
    if (task + 2 < t_end) load_task(b, task + 2, log2S, A);
    if (B.job != cur) {
      finish_job(b, cur, sh);
      cur = B.job;
    }
    accumulate_task(b, B, g8, sh);
  }
  if (cur >= 0) finish_job(b, cur, sh);
}

int refine_grid(int64_t total_tasks) {
  static int occ = 0;
  if (occ <= 0) {
    int blocks = 0;
    const hipError_t e =
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, refine_kernel, kBlock, 0);
    occ = (e == hipSuccess && blocks > 0) ? blocks : 1;
  }
  const int64_t want = (int64_t)device_cu_count() * occ;
  return (int)(total_tasks < want ? total_tasks : want);
}

hipError_t launch_refine(RefineBatch& b, hipStream_t stream) {
  if (b.nblocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(refine_kernel, dim3(b.nblocks), dim3(kBlock), 0, stream, b);
  return hipGetLastError();
}

}  // namespace aaac
