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
// Errors of the assignment (optional). With the cell sums, the total weighted error of the codes
// and selectors under any tables T is
//   E = sum I (w - s T_c[q])^2 = W2 - 2 sum_cells T num + sum_cells T^2 den,   W2 = sum I w^2,
// formed by the last workgroup of the matrix twice: with the tables the codes were chosen with
// (the error after the assign half-step) and with the tables it writes (after this half-step).
// W2 depends only on W and I: the caller either has it from an earlier call (then it costs
// nothing), or every thread sums I w^2 over its weights in a register (exact fp64 terms), one more
// fp64 fma per weight.
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
__device__ __forceinline__ void load_task(const TaskCursor& c, int log2S, int tid, TaskRows& t) {
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
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
                                                int tid, double& w2) {
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

__device__ __forceinline__ void load_task16(const TaskCursor& c, int log2S, int tid,
                                            TaskRows16& t) {
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
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
__device__ __forceinline__ void load_rows(const TaskCursor& c, int log2S, int tid, TaskRows& t) {
  load_task(c, log2S, tid, t);
}
__device__ __forceinline__ void load_rows(const TaskCursor& c, int log2S, int tid, TaskRows16& t) {
  load_task16(c, log2S, tid, t);
}
template <int GL, bool ERRS, int PART>
__device__ __forceinline__ void accumulate_rows(const TaskRows& t, int gl, RefineShared& sh,
                                                int tid, double& w2) {
  accumulate_task<GL, ERRS>(t, gl, sh, tid, w2);
}
template <int GL, bool ERRS, int PART>
__device__ __forceinline__ void accumulate_rows(const TaskRows16& t, int gl, RefineShared& sh,
                                                int tid, double& w2) {
  accumulate_task16<GL, PART, ERRS>(t, gl, sh, tid, w2);
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
// caller's running sum of I w^2, reset here). pt is the group of kBlock threads that accumulates;
// every thread of it calls this (it holds the group's barriers).
template <bool ERRS, class Part>
__device__ void finish_job(const RefineBatch& b, int j, RefineShared& sh, Part pt, double& w2) {
  // ERRS: this call summed I w^2 (w2); b.errs alone: W2 comes from the caller
  const int tid = pt.tid();
  const RefineJob& jb = b.job[j];
  __shared__ double part4[4][kVals];
  __shared__ double w2s[kWavesPerBlock + 1];
  __shared__ uint32_t ticket;
  if (ERRS) {
    // this workgroup's sum of I w^2: lanes by butterfly, waves in order
    const double ws = block_sum_f64_t<kWave>(w2, kWave);
    w2 = 0.0;
    if ((tid & (kWave - 1)) == 0) w2s[tid / kWave] = ws;
  }
  pt.sync();
  {
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
  pt.sync();
#pragma unroll
  for (int k = 0; k < kVals; ++k) sh.bins[k >> 1][k & 1][tid] = 0.0;
  double* part = b.partials + (size_t)j * kPartVals * b.slots;
  const int slot = (int)blockIdx.x - jb.wg_lo;
  if (tid < kVals) {
    const double tot = ((part4[0][tid] + part4[1][tid]) + part4[2][tid]) + part4[3][tid];
    part[(size_t)tid * b.slots + slot] = tot;
    __threadfence();
  }
  if (ERRS && tid == kVals) {
    part[(size_t)kW2 * b.slots + slot] = ((w2s[0] + w2s[1]) + w2s[2]) + w2s[3];
    __threadfence();
  }
  pt.sync();
  if (tid == 0) ticket = atomicAdd(b.counters + j, 1u);
  pt.sync();
  if (ticket != (uint32_t)(jb.wg_count - 1)) return;
  // last workgroup of this job: every partial is visible after the fence
  __threadfence();
  {
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
  if (ERRS && (tid & 63) == 0) {
    // the I w^2 partials, quarter q of the workgroups per thread, in workgroup order
    const int q = tid >> 6;
    const int cnt = jb.wg_count;
    const double* pv = part + (size_t)kW2 * b.slots;
    double s = 0.0;
    for (int i = (q * cnt) / 4; i < ((q + 1) * cnt) / 4; ++i) s += pv[i];
    w2s[q] = s;
  }
  pt.sync();
  __shared__ double eterm[2][kCells];
  if (tid < kCells) {
    const int c = tid >> 4, idx = tid & 15;
    const int vn = 2 * tid, vd = 2 * tid + 1;
    const double nsum = ((part4[0][vn] + part4[1][vn]) + part4[2][vn]) + part4[3][vn];
    const double dsum = ((part4[0][vd] + part4[1][vd]) + part4[2][vd]) + part4[3][vd];
    double et = 0.0, en = 0.0;
    if (idx < b.n) {
      const float old = jb.tables_in[c * b.n + idx];
      const double val = dsum > 0.0 ? nsum / dsum : (double)old;
      const float nv = (b.flags & 1) ? f64_to_bf16_value(val) : (float)val;
      jb.tables_out[c * b.n + idx] = nv;
      // this cell's part of the assignment's error, T^2 den - 2 T num, with the old entry and
      // with the entry just written
      const double T = (double)old, Tn = (double)nv;
      et = T * (T * dsum - 2.0 * nsum);
      en = Tn * (Tn * dsum - 2.0 * nsum);
    }
    if (b.errs) {
      eterm[0][tid] = et;
      eterm[1][tid] = en;
    }
  }
  if (b.errs) {
    pt.sync();
    if (tid == 0 && jb.err_out) {
      const double W2 = ERRS ? ((w2s[0] + w2s[1]) + w2s[2]) + w2s[3] : *jb.w2;
      double x = 0.0, y = 0.0;
      for (int k = 0; k < kCells; ++k) {
        x += eterm[0][k];
        y += eterm[1][k];
      }
      jb.err_out[0] = W2 + x;
      jb.err_after[0] = W2 + y;
      if (ERRS) *jb.w2 = W2;
    }
  }
  if (tid == 0) b.counters[j] = 0u;
  pt.sync();
}

}  // namespace

namespace {

// The refine kernel's work for one workgroup, with the bins in sh; pt names the kBlock threads
// that run it. PART: weights of a row whose terms are formed before their adds (accumulate_task16).
template <bool WIDE, int GL, bool ERRS, int PART = 16, class Part = WholeBlock>
__device__ __forceinline__ void refine_body(const RefineBatch& b, RefineShared& sh, Part pt) {
  const int tid = pt.tid();
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
  load_rows(c, log2S, tid, A);
  cursor_next(b, c);
  for (int64_t task = t_begin; task < t_end; task += 2) {
    load_rows(c, log2S, tid, B);
    cursor_next(b, c);
    if (A.job != cur) {
      if (cur >= 0) finish_job<ERRS>(b, cur, sh, pt, w2);
      cur = A.job;
    }
    accumulate_rows<GL, ERRS, PART>(A, gl, sh, tid, w2);
    if (task + 1 >= t_end) break;
    load_rows(c, log2S, tid, A);
    cursor_next(b, c);
    if (B.job != cur) {
      finish_job<ERRS>(b, cur, sh, pt, w2);
      cur = B.job;
    }
    accumulate_rows<GL, ERRS, PART>(B, gl, sh, tid, w2);
  }
  if (cur >= 0) finish_job<ERRS>(b, cur, sh, pt, w2);
}

}  // namespace

template <bool WIDE, int GL, bool ERRS>
__global__ __launch_bounds__(kBlock, 1) void refine_kernel(RefineBatch b) {
  __shared__ RefineShared sh;
  refine_body<WIDE, GL, ERRS>(b, sh, WholeBlock());
}

// ------------------------------------------------------------------------------------------------
// Fused assign + accumulate: one launch per iteration of the loop (AAAC summary §2 mechanism 4,
// the alternation of assignment and refinement).
//
// The refine kernel's grid, task ranges and thread mapping, with the assign step done in place:
// a wave computes the codes and selections of a row from the lookup structure (lookup.h), writes
// them, and adds the row's terms into its bins from the weights it already holds. W is read once
// per iteration instead of twice and the codes are never read back. The bins keep the kernel at
// one workgroup of four waves per CU, so each wave overlaps its own work: the weights of its next
// task load while it runs the current one. Results are bitwise those of the assign launch
// followed by the refine launch: the codes and selections come from the same per-row search, and
// the same threads add the same terms in the same order.
// ------------------------------------------------------------------------------------------------
namespace {

struct FusedShared {
  RefineShared rs;
  Lut lut;
  LutScratch ls;
};

// One task's weights and importances in registers (loads as in load_task16).
struct FusedRows {
  uint4 va[kWideRowsPerWave], vb[kWideRowsPerWave];
  float4 I[4];
  int64_t r0, R, C;
  int c0;
  int job;
  bool active;
};

__device__ __forceinline__ void load_fused(const TaskCursor& c, FusedRows& t) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int c0 = c.slab * kWideSlab + lane * kWideLane;
  const int64_t R = c.R, C = c.C;
  t.active = c0 < C;
  const int64_t cl = t.active ? c0 : 0;
  t.c0 = c0;
  t.job = c.job;
  t.R = R;
  t.C = C;
  t.r0 = c.rb * kWideRowsPerTask + wave;
#pragma unroll
  for (int i = 0; i < kWideRowsPerWave; ++i) {
    int64_t r = t.r0 + (int64_t)kWavesPerBlock * i;
    r = r < R ? r : R - 1;
    const int64_t base = r * C + cl;
    t.va[i] = *reinterpret_cast<const uint4*>(c.W + base);
    t.vb[i] = *reinterpret_cast<const uint4*>(c.W + base + 8);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) t.I[q] = *reinterpret_cast<const float4*>(c.I + cl + 4 * q);
}

// A row whose codes and selections are known and whose terms are not added yet: its adds are
// issued during the next row's search, so that they never sit in the LDS queue in front of that
// row's lookups. A pending row with zero scale and importance adds zeros (nothing changes).
struct Pending {
  float w[16];
  float If[16];
  uint2 cw;                  // chosen codes, nibble m of word h: weight 8h + m
  double sd, s2;             // s and s^2 in fp64 (0 for an inactive lane)
  uint32_t off;              // byte offset of the chosen table's bins
  bool active;
};

constexpr uint32_t kBinRow = sizeof(double) * 2 * kBlock;   // one cell's {num, den} columns

__device__ __forceinline__ void pending_clear(Pending& p) {
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    p.w[k] = 0.0f;
    p.If[k] = 0.0f;
  }
  p.cw = make_uint2(0u, 0u);
  p.sd = 0.0;
  p.s2 = 0.0;
  p.off = 0u;
  p.active = false;
}

// Terms of weight k of the pending row and their adds (the refine kernel's terms and order:
// num, then den, weights in column order).
template <bool ERRS>
__device__ __forceinline__ void pending_add(const Pending& p, int k, char* lds, double& w2) {
  const uint32_t word = k < 8 ? p.cw.x : p.cw.y;
  const uint32_t q = (word >> (4 * (k & 7))) & 15u;
  double* const a = reinterpret_cast<double*>(lds + p.off + q * kBinRow);
  const double Id = (double)p.If[k];
  const double wd = (double)p.w[k];
  atomicAdd(a, Id * (p.sd * wd));
  atomicAdd(a + kBlock, Id * p.s2);
  if (ERRS) w2 = __builtin_fma(p.active ? Id : 0.0, wd * wd, w2);
}

template <bool ERRS>
__device__ __forceinline__ void pending_flush(const Pending& p, char* lds, double& w2) {
#pragma unroll
  for (int k = 0; k < 16; ++k) pending_add<ERRS>(p, k, lds, w2);
}

// One row: the search of row16_core (same arithmetic, so the same codes and selections) with the
// pending row's adds placed between its LDS reads: every record read first, then four of the
// pending adds while they are in flight, then every candidate read, then the decisions with the
// other twelve adds among them. The row then becomes the pending row.
template <int G16, int S16, bool ERRS>
__device__ __forceinline__ void fused_row(const Lut& lut, int n, int g16, int s16, bool active,
                                          const uint16_t* wsafe, const float* isafe,
                                          const uint4& va, const uint4& vb,
                                          const float (&If)[16], Pending& pend, char* lds,
                                          double& w2, Row16& o) {
  float w[16];
  Row16Scale sc;
  row16_scale<G16>(va, vb, g16, w, sc);
  uint32_t rec[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) rec[k] = lut_record(w[k], sc.Y, lut);
#pragma unroll
  for (int k = 0; k < 4; ++k) pending_add<ERRS>(pend, k, lds, w2);
  __builtin_amdgcn_sched_barrier(0);
  float4 cand[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) cand[k] = lut_candidates(rec[k], lut);
  __builtin_amdgcn_sched_barrier(0);
  uint32_t c[16];
  double accd = 0.0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float acc = 0.0f, a0 = 0.0f, a1 = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int kk = 4 * q + k;
      c[kk] = lut_decide<kErrNone>(w[kk], sc.nse, rec[kk], cand[kk], If[kk], acc, a0, a1);
      if (kk < 12) pending_add<ERRS>(pend, kk + 4, lds, w2);
      // keep the adds spread among the decisions
      __builtin_amdgcn_sched_barrier(0);
    }
    accd = (q == 0) ? (double)acc : accd + (double)acc;
  }
  row16_finish<kErrNone, S16>(lut, n, s16, active, wsafe, isafe, c, accd, 0.0, 0.0, sc, o);
  // this row is the next pending row
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    pend.w[k] = w[k];
    pend.If[k] = If[k];
  }
  pend.cw = chosen_codes16(o);
  pend.sd = active ? (double)o.s : 0.0;   // fp64 terms: exact for every bf16 scale
  pend.s2 = pend.sd * pend.sd;
  pend.off = o.sel ? 16u * kBinRow : 0u;
  pend.active = active;
}

// Every row of one task (rows past the end are the same for the whole wave and are skipped).
template <int G16, int S16, bool ERRS>
__device__ __forceinline__ void fused_task(const RefineBatch& b, const FusedRows& t,
                                           FusedShared& sh, int g16, int s16, int log2S,
                                           Pending& pend, double& w2) {
  const RefineJob& jb = b.job[t.job];
  const float If[16] = {t.I[0].x, t.I[0].y, t.I[0].z, t.I[0].w, t.I[1].x, t.I[1].y,
                        t.I[1].z, t.I[1].w, t.I[2].x, t.I[2].y, t.I[2].z, t.I[2].w,
                        t.I[3].x, t.I[3].y, t.I[3].z, t.I[3].w};
  const int cl = t.active ? t.c0 : 0;
  char* const lds = reinterpret_cast<char*>(&sh.rs.bins[0][0][0]) + threadIdx.x * sizeof(double);
#pragma unroll
  for (int i = 0; i < kWideRowsPerWave; ++i) {
    const int64_t r = t.r0 + (int64_t)kWavesPerBlock * i;
    if (r >= t.R) break;
    const int64_t rc = r * t.C;               // wave-uniform; a multiple of S
    Row16 o;
    fused_row<G16, S16, ERRS>(sh.lut, b.n, g16, s16, t.active, jb.W + rc + cl, jb.I + cl,
                              t.va[i], t.vb[i], If, pend, lds, w2, o);
    if (t.active) {
      *reinterpret_cast<uint2*>(jb.codes_out + (rc >> 3) + (t.c0 >> 3)) = pend.cw;
      if (((t.c0 >> 4) & (s16 - 1)) == 0) jb.sel_out[(rc >> log2S) + (t.c0 >> log2S)] = (uint8_t)o.sel;
    }
  }
}

}  // namespace

template <int G16, int S16, bool ERRS>
__global__ __launch_bounds__(kBlock, 1) void assign_refine_kernel(RefineBatch b) {
  __shared__ FusedShared sh;
  const int tid = threadIdx.x;
  const int g16 = b.g / kWideLane, s16 = b.S / kWideLane;
  const int log2S = 31 - __builtin_clz((unsigned)b.S);
#pragma unroll
  for (int k = 0; k < kVals; ++k) sh.rs.bins[k >> 1][k & 1][tid] = 0.0;
  const int64_t t_begin = task_lo(blockIdx.x, b.total_tasks, gridDim.x);
  const int64_t t_end = task_lo(blockIdx.x + 1, b.total_tasks, gridDim.x);
  if (t_begin >= t_end) return;
  // two statically named buffers, as in the refine kernel: task t + 1 loads while t runs
  FusedRows A, B;
  int cur = -1;
  double w2 = 0.0;
  char* const lds = reinterpret_cast<char*>(&sh.rs.bins[0][0][0]) + tid * sizeof(double);
  Pending pend;
  pending_clear(pend);
  TaskCursor c;
  cursor_init(b, t_begin, t_end - 1, c);
  load_fused(c, A);
  cursor_next(b, c);
  for (int64_t task = t_begin; task < t_end; task += 2) {
    load_fused(c, B);
    cursor_next(b, c);
    if (A.job != cur) {
      // the pending row belongs to the matrix being left. The last barrier of finish_job (or the
      // kernel's start) orders the rebuild after every wave's last use of the previous lookup
      // structure.
      if (cur >= 0) {
        pending_flush<ERRS>(pend, lds, w2);
        pending_clear(pend);
        finish_job<ERRS>(b, cur, sh.rs, WholeBlock(), w2);
      }
      build_lut<kBlock>(b.job[A.job].tables_in, b.n, sh.lut, sh.ls);
      cur = A.job;
    }
    fused_task<G16, S16, ERRS>(b, A, sh, g16, s16, log2S, pend, w2);
    if (task + 1 >= t_end) break;
    load_fused(c, A);
    cursor_next(b, c);
    if (B.job != cur) {
      pending_flush<ERRS>(pend, lds, w2);
      pending_clear(pend);
      finish_job<ERRS>(b, cur, sh.rs, WholeBlock(), w2);
      build_lut<kBlock>(b.job[B.job].tables_in, b.n, sh.lut, sh.ls);
      cur = B.job;
    }
    fused_task<G16, S16, ERRS>(b, B, sh, g16, s16, log2S, pend, w2);
  }
  pending_flush<ERRS>(pend, lds, w2);
  finish_job<ERRS>(b, cur, sh.rs, WholeBlock(), w2);
}

namespace {

template <bool ERRS>
hipError_t launch_assign_refine_t(RefineBatch& b, hipStream_t stream) {
  const dim3 grid(b.nblocks), block(kBlock);
  const int g16 = b.g / kWideLane, s16 = b.S / kWideLane;
  if (g16 == 8 && s16 == 8)
    hipLaunchKernelGGL((assign_refine_kernel<8, 8, ERRS>), grid, block, 0, stream, b);
  else if (g16 == 8 && s16 == 1)
    hipLaunchKernelGGL((assign_refine_kernel<8, 1, ERRS>), grid, block, 0, stream, b);
  else if (g16 == 1 && s16 == 1)
    hipLaunchKernelGGL((assign_refine_kernel<1, 1, ERRS>), grid, block, 0, stream, b);
  else
    hipLaunchKernelGGL((assign_refine_kernel<0, 0, ERRS>), grid, block, 0, stream, b);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_assign_refine(RefineBatch& b, hipStream_t stream) {
  if (b.nblocks <= 0) return hipSuccess;
  // the I w^2 sum only when the caller does not have it
  if (b.errs && !(b.flags & 2)) return launch_assign_refine_t<true>(b, stream);
  return launch_assign_refine_t<false>(b, stream);
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
