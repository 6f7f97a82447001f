// Refine step (AAAC summary §2 mechanism 4): activation-weighted k-means update of both tables.
//
// For every cell (table c, entry j) the kernel sums num = sum I_k s w_k and den = sum I_k s^2 over
// the weights whose selection group chose c and whose code is j; the new entry is num / den (the
// minimizer of sum I (w - s t)^2), or the old entry if the cell is empty.
//
// Accumulation: each term is exact in fp64 for every finite input (s w and s^2 are products of two
// bf16 values, at most 16 significant bits, formed in fp64, times the 24-bit I; the exponents stay
// far inside the fp64 range), and every thread adds its terms into a private column of 64 fp64 bins in LDS
// (32 cells x {num, den}, laid out [bin][thread]) with ds_add_f64. When a workgroup leaves a matrix
// it reduces its 256 columns in a fixed order and writes one fp64 partial per (bin, workgroup); the
// last workgroup to finish that matrix (an integer ticket) adds the partials in workgroup order and
// divides. Every order is fixed, so results are bitwise reproducible.
//
// The bins take 128 KB, one workgroup per CU; to keep enough bytes in flight each wave loads the
// rows of its next task before it accumulates the current one.
//
// Error of the incoming assignment (optional). With the cell sums, the total weighted error of the
// codes and selectors under the tables they were chosen with is
//   E = sum I (w - s T_c[q])^2 = W2 - 2 sum_cells T num + sum_cells T^2 den,   W2 = sum I w^2,
// formed by the last workgroup of the matrix before it writes the new tables. W2 depends only on
// W and I: the caller either has it from an earlier call (then it costs nothing), or every thread
// sums I w^2 over its weights in a register (exact fp64 terms), one more fp64 fma per weight.
#include <type_traits>

#include "common.h"
#include "lookup.h"

namespace aaac {

namespace {

constexpr int kCells = 32;   // 2 tables x 16 entries
constexpr int kVals = 64;    // value v = 2 cell + {0: num, 1: den}
constexpr int kW2 = 64;      // partial value 64: sum I w^2 (with error output)

// bins[cell][sum][thread]: a thread's num and den of one cell are 2 KB apart (one immediate
// offset), and the 64 lanes of a wave touch 64 consecutive doubles (no bank conflicts).
struct RefineShared {
  double bins[kCells][2][kBlock];
};

// Position of the next task to load, kept in scalar registers. The fields of a matrix are read
// from the kernel arguments only when the cursor enters it: scalar memory reads share a wait
// counter with LDS operations, so reading them for every task would make the wave wait for all of
// its LDS adds in flight. Row block and slab advance by counting instead of dividing.
struct TaskCursor {
  int64_t task;          // the task the next load reads
  int64_t last;          // last task of this workgroup: the cursor stops there
  int64_t job_end;       // first task past the current matrix
  int64_t rb;            // row block of `task`
  int64_t R, C;
  int32_t slab, nslab;
  int32_t job;
  const uint16_t* W;
  const float* I;
  const uint32_t* codes;
  const uint8_t* sel;
};

__device__ __forceinline__ void cursor_enter(const RefineBatch& b, int j, TaskCursor& c) {
  const RefineJob& jb = b.job[j];
  c.job = j;
  c.job_end = jb.geom.task_begin + jb.geom.ntasks;
  c.nslab = jb.geom.nslab;
  c.R = jb.geom.R;
  c.C = jb.geom.C;
  c.W = jb.W;
  c.I = jb.I;
  c.codes = jb.codes;
  c.sel = jb.sel;
}

__device__ __forceinline__ void cursor_init(const RefineBatch& b, int64_t task, int64_t last,
                                            TaskCursor& c) {
  int j = 0;
  while (j + 1 < b.njobs && task >= b.job[j + 1].geom.task_begin) ++j;
  cursor_enter(b, j, c);
  c.task = task;
  c.last = last;
  const int64_t local = task - b.job[j].geom.task_begin;
  c.rb = local / c.nslab;
  c.slab = (int32_t)(local - c.rb * c.nslab);
}

__device__ __forceinline__ void cursor_next(const RefineBatch& b, TaskCursor& c) {
  if (c.task >= c.last) return;
  ++c.task;
  if (c.task >= c.job_end) {
    cursor_enter(b, c.job + 1, c);
    c.rb = 0;
    c.slab = 0;
  } else if (++c.slab == c.nslab) {
    c.slab = 0;
    ++c.rb;
  }
}

struct TaskRows {
  uint4 v[kRowsPerWave];
  uint32_t cw[kRowsPerWave];
  uint32_t sb[kRowsPerWave];
  float4 I0, I1;
  int64_t r0;
  int64_t R;
  int job;
  bool active;
};

// Issue every load of one task without branches: a lane past the last column, or a row past the
// last row, reads an in-bounds element of the same matrix instead, and its contribution is dropped
// where it is used (zero importance for the lane; rows past the end are skipped). Loads that are
// never conditional let the compiler wait for exactly the task being used while later tasks' loads
// stay in flight.
__device__ __forceinline__ void load_task(const TaskCursor& c, int log2S, TaskRows& t) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int c0 = c.slab * kSlab + lane * kPerLane;
  const int64_t R = c.R, C = c.C;
  const int64_t rb = c.rb;
  const int j = c.job;
  t.active = c0 < C;
  const int64_t cl = t.active ? c0 : 0;
  t.job = j;
  t.R = R;
  t.r0 = rb * kRowsPerTask + wave;
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    int64_t r = t.r0 + (int64_t)kWavesPerBlock * i;
    r = r < R ? r : R - 1;
    const int64_t base = r * C + cl;
    t.v[i] = *reinterpret_cast<const uint4*>(c.W + base);
    t.cw[i] = c.codes[base >> 3];
    t.sb[i] = c.sel[base >> log2S];
  }
  t.I0 = *reinterpret_cast<const float4*>(c.I + cl);
  t.I1 = *reinterpret_cast<const float4*>(c.I + cl + 4);
}

template <int G8, bool ERRS>
__device__ __forceinline__ void accumulate_task(const TaskRows& t, int g8, RefineShared& sh,
                                                double& w2) {
  const int tid = threadIdx.x;
  const float If[8] = {t.I0.x, t.I0.y, t.I0.z, t.I0.w, t.I1.x, t.I1.y, t.I1.z, t.I1.w};
  double Id[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) Id[k] = (double)If[k];
  char* const lds = reinterpret_cast<char*>(&sh.bins[0][0][0]) + tid * sizeof(double);
  // the scales of all rows first: eight independent lane reductions. A lane past the last column
  // reads a group of its own matrix and gets scale 0, so its terms are zero (whole scale groups are
  // inactive together, so no active group sees the zero).
  float s[kRowsPerWave];
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    const float si = __uint_as_float(block_max_u32_t<G8>(lane_absmax_bits(t.v[i]), g8) << 16);
    s[i] = t.active ? si : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    // rows past the end of the matrix are the same for the whole wave
    if (t.r0 + (int64_t)kWavesPerBlock * i >= t.R) break;
    // s w and s^2 are formed in fp64: products of two bf16 values (16 significant bits) are
    // exact there for every finite bf16 scale, and so are their products with the fp32 I
    const double sd = (double)s[i];
    const double s2 = sd * sd;
    float w[8];
    unpack8(t.v[i], w);
    char* const row = lds + (t.sb[i] ? 16 * sizeof(sh.bins[0]) : 0);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t q = (t.cw[i] >> (4 * k)) & 15u;
      double* const p = reinterpret_cast<double*>(row + q * sizeof(sh.bins[0]));
      const double wd = (double)w[k];
      atomicAdd(p, Id[k] * (sd * wd));
      atomicAdd(p + kBlock, Id[k] * s2);
      if (ERRS) w2 = __builtin_fma(Id[k] * (t.active ? 1.0 : 0.0), wd * wd, w2);
    }
    // one row at a time: interleaving rows would push the live registers past the 256 a lane can
    // address and spill loaded values that are still in flight
    __builtin_amdgcn_sched_barrier(0);
  }
}

struct TaskRows16 {
  uint4 va[kWideRowsPerWave], vb[kWideRowsPerWave];
  uint2 cw[kWideRowsPerWave];
  uint32_t sb[kWideRowsPerWave];
  float4 I[4];
  int64_t r0;
  int64_t R;
  int job;
  bool active;
};

__device__ __forceinline__ void load_task16(const TaskCursor& c, int log2S, TaskRows16& t) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int c0 = c.slab * kWideSlab + lane * kWideLane;
  const int64_t R = c.R, C = c.C;
  const int64_t rb = c.rb;
  const int j = c.job;
  t.active = c0 < C;
  const int64_t cl = t.active ? c0 : 0;
  t.job = j;
  t.R = R;
  t.r0 = rb * kWideRowsPerTask + wave;
#pragma unroll
  for (int i = 0; i < kWideRowsPerWave; ++i) {
    int64_t r = t.r0 + (int64_t)kWavesPerBlock * i;
    r = r < R ? r : R - 1;
    const int64_t base = r * C + cl;
    t.va[i] = *reinterpret_cast<const uint4*>(c.W + base);
    t.vb[i] = *reinterpret_cast<const uint4*>(c.W + base + 8);
    t.cw[i] = *reinterpret_cast<const uint2*>(c.codes + (base >> 3));
    t.sb[i] = c.sel[base >> log2S];
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) t.I[q] = *reinterpret_cast<const float4*>(c.I + cl + 4 * q);
}

// col: this thread's column of bins (its index among the accumulating threads). PART: weights
// whose terms are formed before their adds are issued (16: the whole row; 8: half a row, for
// kernels that must keep registers low). The adds go out in the same order either way.
template <int G16, int PART = 16, bool ERRS = false>
__device__ __forceinline__ void accumulate_task16(const TaskRows16& t, int g16, RefineShared& sh,
                                                  int col, double& w2) {
  const int tid = col;
  const float If[16] = {t.I[0].x, t.I[0].y, t.I[0].z, t.I[0].w, t.I[1].x, t.I[1].y,
                        t.I[1].z, t.I[1].w, t.I[2].x, t.I[2].y, t.I[2].z, t.I[2].w,
                        t.I[3].x, t.I[3].y, t.I[3].z, t.I[3].w};
  char* const lds = reinterpret_cast<char*>(&sh.bins[0][0][0]) + tid * sizeof(double);
#pragma unroll
  for (int i = 0; i < kWideRowsPerWave; ++i) {
    if (t.r0 + (int64_t)kWavesPerBlock * i >= t.R) break;
    float w[16];
    unpack8(t.va[i], *reinterpret_cast<float(*)[8]>(&w[0]));
    unpack8(t.vb[i], *reinterpret_cast<float(*)[8]>(&w[8]));
    // the group scale; a lane past the last column gets scale 0, so its terms are zero (see
    // accumulate_task)
    const float si = __uint_as_float(block_max_u32_t<G16>(absmax16_f32_bits(w), g16));
    const double sd = t.active ? (double)si : 0.0;   // fp64 terms: exact for every bf16 scale
    const double s2 = sd * sd;
    char* const row = lds + (t.sb[i] ? 16 * sizeof(sh.bins[0]) : 0);
    // every term of the row first, then every add: with one wave per SIMD, an add issued right
    // after the multiply that feeds it would wait for that result
#pragma unroll
    for (int h = 0; h < 16; h += PART) {
      double num[PART], den[PART];
      double* p[PART];
#pragma unroll
      for (int u = 0; u < PART; ++u) {
        const int k = h + u;
        const uint32_t word = k < 8 ? t.cw[i].x : t.cw[i].y;
        const uint32_t q = (word >> (4 * (k & 7))) & 15u;
        p[u] = reinterpret_cast<double*>(row + q * sizeof(sh.bins[0]));
        const double Id = (double)If[k];
        const double wd = (double)w[k];
        num[u] = Id * (sd * wd);
        den[u] = Id * s2;
        // a lane past the last column reads a weight of its own matrix: it adds nothing
        if (ERRS) w2 = __builtin_fma(t.active ? Id : 0.0, wd * wd, w2);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < PART; ++u) {
        atomicAdd(p[u], num[u]);
        atomicAdd(p[u] + kBlock, den[u]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// The two task layouts behind one name each, chosen by the buffer type.
__device__ __forceinline__ void load_rows(const TaskCursor& c, int log2S, TaskRows& t) {
  load_task(c, log2S, t);
}
__device__ __forceinline__ void load_rows(const TaskCursor& c, int log2S, TaskRows16& t) {
  load_task16(c, log2S, t);
}
template <int GL, bool ERRS>
__device__ __forceinline__ void accumulate_rows(const TaskRows& t, int gl, RefineShared& sh,
                                                double& w2) {
  accumulate_task<GL, ERRS>(t, gl, sh, w2);
}
template <int GL, bool ERRS>
__device__ __forceinline__ void accumulate_rows(const TaskRows16& t, int gl, RefineShared& sh,
                                                double& w2) {
  accumulate_task16<GL, 16, ERRS>(t, gl, sh, threadIdx.x, w2);
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
// all partials and writes the tables (and with ERRS the error of the incoming assignment; w2 is the
// caller's running sum of I w^2, reset here). Every thread of the workgroup calls it (it holds
// barriers); tid is the caller's index among the kBlock accumulating threads, and threads outside
// [0, kBlock) only take part in the barriers.
template <bool ERRS>
__device__ void finish_job(const RefineBatch& b, int j, RefineShared& sh, int tid, double& w2) {
  // ERRS: this call summed I w^2 (w2); b.errs alone: W2 comes from the caller
  const bool act = tid >= 0 && tid < kBlock;
  const RefineJob& jb = b.job[j];
  __shared__ double part4[4][kVals];
  __shared__ double w2s[kWavesPerBlock + 1];
  __shared__ uint32_t ticket;
  if (ERRS) {
    // this workgroup's sum of I w^2: lanes by butterfly, waves in order
    const double ws = block_sum_f64_t<kWave>(act ? w2 : 0.0, kWave);
    w2 = 0.0;
    if (act && (tid & (kWave - 1)) == 0) w2s[tid / kWave] = ws;
  }
  __syncthreads();
  if (act) {
    // value v = tid & 63 over the 64 columns of quarter q = tid >> 6: four interleaved sums over a
    // rotated column order (no bank conflicts), all reads issued before the adds, combined in a
    // fixed order
    const int v = tid & 63, q = tid >> 6;
    const double* col = &sh.bins[v >> 1][v & 1][q * 64];
    double a[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int i = 0; i < 64; ++i) a[i & 3] += col[(i + v) & 63];
    part4[q][v] = (a[0] + a[1]) + (a[2] + a[3]);
  }
  __syncthreads();
  if (act) {
#pragma unroll
    for (int k = 0; k < kVals; ++k) sh.bins[k >> 1][k & 1][tid] = 0.0;
  }
  double* part = b.partials + (size_t)j * kPartVals * b.slots;
  const int slot = (int)blockIdx.x - jb.wg_lo;
  if (act && tid < kVals) {
    const double tot = ((part4[0][tid] + part4[1][tid]) + part4[2][tid]) + part4[3][tid];
    part[(size_t)tid * b.slots + slot] = tot;
    __threadfence();
  }
  if (ERRS && act && tid == kVals) {
    part[(size_t)kW2 * b.slots + slot] = ((w2s[0] + w2s[1]) + w2s[2]) + w2s[3];
    __threadfence();
  }
  __syncthreads();
  if (tid == 0) ticket = atomicAdd(b.counters + j, 1u);
  __syncthreads();
  if (ticket != (uint32_t)(jb.wg_count - 1)) return;
  // last workgroup of this job: every partial is visible after the fence
  __threadfence();
  if (act) {
    // the partials of value v, quarter q of the workgroups: eight loads in flight per step, added
    // in workgroup order
    const int v = tid & 63, q = tid >> 6;
    const int cnt = jb.wg_count;
    const int s0 = (q * cnt) / 4, s1 = ((q + 1) * cnt) / 4;
    const double* pv = part + (size_t)v * b.slots;
    double s = 0.0;
    int i = s0;
    for (; i + 8 <= s1; i += 8) {
      double x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = pv[i + u];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += x[u];
    }
    for (; i < s1; ++i) s += pv[i];
    part4[q][v] = s;
  }
  if (ERRS && act && (tid & 63) == 0) {
    // the I w^2 partials, quarter q of the workgroups per thread, in workgroup order
    const int q = tid >> 6;
    const int cnt = jb.wg_count;
    const double* pv = part + (size_t)kW2 * b.slots;
    double s = 0.0;
    for (int i = (q * cnt) / 4; i < ((q + 1) * cnt) / 4; ++i) s += pv[i];
    w2s[q] = s;
  }
  __syncthreads();
  __shared__ double eterm[kCells];
  if (act && tid < kCells) {
    const int c = tid >> 4, idx = tid & 15;
    const int vn = 2 * tid, vd = 2 * tid + 1;
    const double nsum = ((part4[0][vn] + part4[1][vn]) + part4[2][vn]) + part4[3][vn];
    const double dsum = ((part4[0][vd] + part4[1][vd]) + part4[2][vd]) + part4[3][vd];
    double et = 0.0;
    if (idx < b.n) {
      const float old = jb.tables_in[c * b.n + idx];
      const double val = dsum > 0.0 ? nsum / dsum : (double)old;
      // this cell's part of the incoming error: T^2 den - 2 T num with the old entry T
      const double T = (double)old;
      et = T * (T * dsum - 2.0 * nsum);
      jb.tables_out[c * b.n + idx] = (b.flags & 1) ? f64_to_bf16_value(val) : (float)val;
    }
    if (b.errs) eterm[tid] = et;
  }
  if (b.errs) {
    __syncthreads();
    if (tid == 0 && jb.err_out) {
      const double W2 = ERRS ? ((w2s[0] + w2s[1]) + w2s[2]) + w2s[3] : *jb.w2;
      double x = 0.0;
      for (int k = 0; k < kCells; ++k) x += eterm[k];
      jb.err_out[0] = W2 + x;
      if (ERRS) *jb.w2 = W2;
    }
  }
  if (tid == 0) b.counters[j] = 0u;
  __syncthreads();
}

}  // namespace

template <bool WIDE, int GL, bool ERRS>
__global__ __launch_bounds__(kBlock, 1) void refine_kernel(RefineBatch b) {
  __shared__ RefineShared sh;
  const int tid = threadIdx.x;
  const int gl = b.g / (WIDE ? kWideLane : kPerLane);   // lanes per scale group
  const int log2S = 31 - __builtin_clz((unsigned)b.S);
#pragma unroll
  for (int k = 0; k < kVals; ++k) sh.bins[k >> 1][k & 1][tid] = 0.0;
  const int64_t t_begin = task_lo(blockIdx.x, b.total_tasks, gridDim.x);
  const int64_t t_end = task_lo(blockIdx.x + 1, b.total_tasks, gridDim.x);
  // two statically named buffers: the rows of task t + 1 are in flight while task t accumulates
  typedef typename std::conditional<WIDE, TaskRows16, TaskRows>::type Rows;
  Rows A, B;
  int cur = -1;
  double w2 = 0.0;
  if (t_begin >= t_end) return;
  // the cursor stops at the last task: past the end a buffer reloads that task and is never used
  TaskCursor c;
  cursor_init(b, t_begin, t_end - 1, c);
  load_rows(c, log2S, A);
  cursor_next(b, c);
  for (int64_t task = t_begin; task < t_end; task += 2) {
    load_rows(c, log2S, B);
    cursor_next(b, c);
    if (A.job != cur) {
      if (cur >= 0) finish_job<ERRS>(b, cur, sh, threadIdx.x, w2);
      cur = A.job;
    }
    accumulate_rows<GL, ERRS>(A, gl, sh, w2);
    if (task + 1 >= t_end) break;
    load_rows(c, log2S, A);
    cursor_next(b, c);
    if (B.job != cur) {
      finish_job<ERRS>(b, cur, sh, threadIdx.x, w2);
      cur = B.job;
    }
    accumulate_rows<GL, ERRS>(B, gl, sh, w2);
  }
  if (cur >= 0) finish_job<ERRS>(b, cur, sh, threadIdx.x, w2);
}

// ------------------------------------------------------------------------------------------------
// Fused assign + accumulate: one launch per iteration of the loop (AAAC summary §2 mechanism 4,
// the alternation of assignment and refinement).
//
// A workgroup of 16 waves: 12 assign waves and 4 accumulate waves, one workgroup per CU (the
// accumulate waves hold the 128 KB of bins). The workgroup walks the same task range as a refine
// workgroup, in steps of up to three tasks of one matrix. In step s the assign waves run the assign
// of step s's tasks (four waves per task, the thread mapping of the assign kernel) and write codes
// and selectors; the accumulate waves add up step s - 1 exactly as the refine kernel does (same
// thread per column, same task and row order, same finish), reading the codes just written from
// L2 and the selectors from LDS. Assign and accumulate waves share each SIMD, so one's VALU work
// overlaps the other's LDS adds. Results are bitwise those of the assign launch followed by the
// refine launch.
// ------------------------------------------------------------------------------------------------
constexpr int kFusedAssignWaves = 12;
constexpr int kFusedGroups = kFusedAssignWaves / kWavesPerBlock;          // tasks per step
constexpr int kFusedThreads = (kFusedAssignWaves + kWavesPerBlock) * kWave;
constexpr int kFusedAcc0 = kFusedAssignWaves * kWave;                    // first accumulate thread

namespace {

struct FusedShared {
  RefineShared rs;
  Lut lut;
  LutScratch ls;
  // selector of each (task of the step, row of the task, lane) as written by the assign waves;
  // two copies, for the step being assigned and the step being accumulated
  uint8_t sig[2][kFusedGroups][kWideRowsPerTask][kWave];
};

// Tasks [lo, hi) of the step starting at `task`: up to kFusedGroups tasks, all of one matrix.
__device__ __forceinline__ void fused_step(const RefineBatch& b, int64_t task, int64_t t_end,
                                           int& job, int64_t& hi) {
  int j = 0;
  while (j + 1 < b.njobs && task >= b.job[j + 1].geom.task_begin) ++j;
  const int64_t job_end = b.job[j].geom.task_begin + b.job[j].geom.ntasks;
  hi = task + kFusedGroups;
  hi = hi < job_end ? hi : job_end;
  hi = hi < t_end ? hi : t_end;
  job = j;
}

template <int G16, int S16>
__device__ __forceinline__ void fused_assign_task(const RefineBatch& b, const RefineJob& jb,
                                                  int64_t task, int w, int buf, int grp,
                                                  const Lut& lut, FusedShared& sh) {
  const int lane = threadIdx.x & (kWave - 1);
  const int g16 = b.g / kWideLane, s16 = b.S / kWideLane, n = b.n;
  const int log2S = 31 - __builtin_clz((unsigned)b.S);
  const int64_t local = task - jb.geom.task_begin;
  const int64_t rb = local / jb.geom.nslab;
  const int slab = (int)(local - rb * jb.geom.nslab);
  const int c0 = slab * kWideSlab + lane * kWideLane;
  const bool active = c0 < jb.geom.C;
  const int cl = active ? c0 : 0;
  const int64_t R = jb.geom.R, C = jb.geom.C;
  const int64_t r0 = rb * kWideRowsPerTask + w;
  uint4 va[kWideRowsPerWave], vb[kWideRowsPerWave];
#pragma unroll
  for (int i = 0; i < kWideRowsPerWave; ++i) {
    int64_t r = r0 + (int64_t)kWavesPerBlock * i;
    r = r < R ? r : R - 1;
    const uint16_t* p = jb.W + r * C;
    va[i] = *reinterpret_cast<const uint4*>(p + cl);
    vb[i] = *reinterpret_cast<const uint4*>(p + cl + 8);
  }
  float Ik[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 x = *reinterpret_cast<const float4*>(jb.I + cl + 4 * q);
    Ik[4 * q] = x.x; Ik[4 * q + 1] = x.y; Ik[4 * q + 2] = x.z; Ik[4 * q + 3] = x.w;
  }
#pragma unroll
  for (int i = 0; i < kWideRowsPerWave; ++i) {
    const int64_t r = r0 + (int64_t)kWavesPerBlock * i;
    if (r >= R) break;
    Row16 o;
    row16_core<kErrNone, G16, S16>(lut, n, g16, s16, active, jb.W + r * C + cl, jb.I + cl, va[i],
                                vb[i], Ik, o);
    const int64_t rc = r * C;
    if (active)
      store_row16<kErrNone>(o, jb.codes_out + (rc >> 3), jb.sel_out + (rc >> log2S), nullptr, s16,
                         log2S, c0);
    sh.sig[buf][grp][w + kWavesPerBlock * i][lane] = (uint8_t)o.sel;
  }
}

// The accumulate side of one task: wave w of the accumulate waves adds rows w, w + 4, ... exactly
// as the refine kernel's wave w does, with the selectors from LDS.
template <int G16>
__device__ __forceinline__ void fused_accumulate_task(const RefineBatch& b, const RefineJob& jb,
                                                      int j, int64_t task, int w, int buf,
                                                      int grp, FusedShared& sh) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t local = task - jb.geom.task_begin;
  const int64_t rb = local / jb.geom.nslab;
  const int slab = (int)(local - rb * jb.geom.nslab);
  TaskRows16 t;
  const int c0 = slab * kWideSlab + lane * kWideLane;
  const int64_t R = jb.geom.R, C = jb.geom.C;
  t.active = c0 < C;
  const int cl = t.active ? c0 : 0;
  t.job = j;
  t.R = R;
  t.r0 = rb * kWideRowsPerTask + w;
#pragma unroll
  for (int i = 0; i < kWideRowsPerWave; ++i) {
    int64_t r = t.r0 + (int64_t)kWavesPerBlock * i;
    r = r < R ? r : R - 1;
    const int64_t base = r * C + cl;
    t.va[i] = *reinterpret_cast<const uint4*>(jb.W + base);
    t.vb[i] = *reinterpret_cast<const uint4*>(jb.W + base + 8);
    t.cw[i] = *reinterpret_cast<const uint2*>(jb.codes_out + (base >> 3));
    t.sb[i] = sh.sig[buf][grp][w + kWavesPerBlock * i][lane];
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) t.I[q] = *reinterpret_cast<const float4*>(jb.I + cl + 4 * q);
  double w2 = 0.0;
  accumulate_task16<G16, 8>(t, b.g / kWideLane, sh.rs, (int)threadIdx.x - kFusedAcc0, w2);
}

}  // namespace

template <int G16, int S16>
__global__ __launch_bounds__(kFusedThreads, 1) void assign_refine_kernel(RefineBatch b) {
  __shared__ FusedShared sh;
  const int tid = threadIdx.x;
  const int wave = wave_index();
  const bool acc_wave = wave >= kFusedAssignWaves;
  const int atid = tid - kFusedAcc0;                   // index among the accumulating threads
  if (acc_wave) {
#pragma unroll
    for (int k = 0; k < kVals; ++k) sh.rs.bins[k >> 1][k & 1][atid] = 0.0;
  }
  const int64_t t_begin = task_lo(blockIdx.x, b.total_tasks, gridDim.x);
  const int64_t t_end = task_lo(blockIdx.x + 1, b.total_tasks, gridDim.x);
  int lut_job = -1, acc_job = -1;
  double w2_unused = 0.0;
  int prev_job = -1;
  int64_t prev_lo = 0, prev_hi = 0;                    // the step the accumulate waves take next
  int buf = 0;
  for (int64_t lo = t_begin;; buf ^= 1) {
    int job = -1;
    int64_t hi = lo;
    if (lo < t_end) fused_step(b, lo, t_end, job, hi);
    if (job < 0 && prev_job < 0) break;
    // matrix changes, with every thread: the accumulate side finishes its matrix before it starts
    // the next one; the assign side builds the lookup structure of its new matrix
    if (prev_job >= 0 && prev_job != acc_job) {
      if (acc_job >= 0) finish_job<false>(b, acc_job, sh.rs, atid, w2_unused);
      acc_job = prev_job;
    }
    if (job >= 0 && job != lut_job) {
      __syncthreads();
      build_lut<kFusedThreads>(b.job[job].tables_in, b.n, sh.lut, sh.ls);
      lut_job = job;
    }
    if (!acc_wave) {
      const int grp = wave / kWavesPerBlock;
      if (job >= 0 && lo + grp < hi)
        fused_assign_task<G16, S16>(b, b.job[job], lo + grp, wave % kWavesPerBlock, buf, grp,
                                    sh.lut, sh);
    } else if (prev_job >= 0) {
      // the codes of step s - 1 were written by this workgroup's assign waves before the last
      // barrier (a workgroup-scope release and acquire: all waves share this CU's write-through
      // cache, so a line cached earlier cannot hide them)
      for (int64_t t = prev_lo; t < prev_hi; ++t)
        fused_accumulate_task<G16>(b, b.job[prev_job], prev_job, t, wave - kFusedAssignWaves,
                                   buf ^ 1, (int)(t - prev_lo), sh);
    }
    __syncthreads();
    prev_job = job;
    prev_lo = lo;
    prev_hi = hi;
    lo = hi;
  }
  if (acc_job >= 0) finish_job<false>(b, acc_job, sh.rs, atid, w2_unused);
}

hipError_t launch_assign_refine(RefineBatch& b, hipStream_t stream) {
  if (b.nblocks <= 0) return hipSuccess;
  const dim3 grid(b.nblocks), block(kFusedThreads);
  const int g16 = b.g / kWideLane, s16 = b.S / kWideLane;
  if (g16 == 8 && s16 == 8)
    hipLaunchKernelGGL((assign_refine_kernel<8, 8>), grid, block, 0, stream, b);
  else if (g16 == 8 && s16 == 1)
    hipLaunchKernelGGL((assign_refine_kernel<8, 1>), grid, block, 0, stream, b);
  else if (g16 == 1 && s16 == 1)
    hipLaunchKernelGGL((assign_refine_kernel<1, 1>), grid, block, 0, stream, b);
  else
    hipLaunchKernelGGL((assign_refine_kernel<0, 0>), grid, block, 0, stream, b);
  return hipGetLastError();
}

MatrixGeom refine_geom(int64_t R, int64_t C, int64_t task_begin, int S) {
  return S >= kWideLane ? make_geom(R, C, task_begin, kWideSlab, kWideRowsPerTask)
                        : make_geom(R, C, task_begin);
}

// The bins fill most of the LDS: one workgroup per CU.
int refine_grid(int64_t total_tasks) {
  const int64_t want = (int64_t)device_cu_count();
  return (int)(total_tasks < want ? total_tasks : want);
}

template <bool ERRS>
hipError_t launch_refine_t(RefineBatch& b, hipStream_t stream) {
  const dim3 grid(b.nblocks), block(kBlock);
  if (b.S >= kWideLane) {
    const int g16 = b.g / kWideLane;
    if (g16 == 8)
      hipLaunchKernelGGL((refine_kernel<true, 8, ERRS>), grid, block, 0, stream, b);
    else if (g16 == 1)
      hipLaunchKernelGGL((refine_kernel<true, 1, ERRS>), grid, block, 0, stream, b);
    else
      hipLaunchKernelGGL((refine_kernel<true, 0, ERRS>), grid, block, 0, stream, b);
  } else {
    hipLaunchKernelGGL((refine_kernel<false, 0, ERRS>), grid, block, 0, stream, b);
  }
  return hipGetLastError();
}

hipError_t launch_refine(RefineBatch& b, hipStream_t stream) {
  if (b.nblocks <= 0) return hipSuccess;
  // the I w^2 sum only when the caller does not have it
  if (b.errs && !(b.flags & 2)) return launch_refine_t<true>(b, stream);
  return launch_refine_t<false>(b, stream);
}

}  // namespace aaac
