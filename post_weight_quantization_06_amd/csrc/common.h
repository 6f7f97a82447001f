// Shared definitions of the gfx950 kernels: lane mapping, bf16 helpers, job descriptors and the
// host-side launchers that the C ABI (abi.hip) calls after validating its arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace aaac {

// ------------------------------------------------------------------------------------------------
// Lane mapping shared by the streaming kernels. A wave covers one "slab" of 512 consecutive columns
// of a row: lane l owns columns [slab*512 + 8l, slab*512 + 8l + 8), i.e. one 16-byte load of bf16.
// A workgroup of four waves walks kRowsPerTask rows of one slab (one "task"); tasks are numbered
// row-block-major so that consecutive tasks read consecutive memory.
// ------------------------------------------------------------------------------------------------
constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kPerLane = 8;
constexpr int kSlab = kWave * kPerLane;
constexpr int kRowsPerWave = 8;
constexpr int kRowsPerTask = kRowsPerWave * kWavesPerBlock;

// Wide mapping for selection groups of at least 16 weights: a lane holds 16 consecutive weights
// (two 16-byte loads), a wave row covers 1024 columns, a task is 16 rows x 1024 columns (four rows
// per wave). The per-row work (scale, selection sum, code compaction) is spread over twice as many
// weights as in the 8-weight mapping.
constexpr int kWideLane = 16;
constexpr int kWideSlab = kWave * kWideLane;
constexpr int kWideRowsPerWave = 4;
constexpr int kWideRowsPerTask = kWideRowsPerWave * kWavesPerBlock;

constexpr int kMaxJobs = 8;

// ------------------------------------------------------------------------------------------------
// Nearest-entry lookup structure (built in LDS by the assign kernel from the two tables).
// u in [-1, 1] maps to record rho = round(kLutScale (u + 1)) + 1 through one fma,
//   t = fma(w, Y, kLutMagic),  Y = kLutY / s,  kLutY = kLutScale * 2^-22,
// which lands t in [2, 4), where the fp32 quantum is 2^-22: the low mantissa bits of t hold rho
// (rounded to nearest even, as for any fp32 result), and the exponent field is 128, so shifting the
// bit pattern left by two drops the exponent and leaves 4 rho, the record's byte offset. Record rho
// covers u in [(rho - 1.5) / kLutScale - 1, (rho - 0.5) / kLutScale - 1]. For each table the record
// holds the byte offset of a candidate pair {T[i], T[i+1]} in a small pair array (T[n] reads as
// +inf), valid over that interval widened by kLutSlack: the nearest entry there is T[i], or T[i+1]
// past the one midpoint the record contains. A record that would need other candidates points at a
// NaN pair, which routes its group to the exact full scan. One 32-bit word per record (pair offsets
// of both tables and the code base i0 | i1 << 4) and two 18-pair arrays: a few KB of LDS, and the
// pair reads hit at most 18 distinct addresses per wave, so they never conflict.
// ------------------------------------------------------------------------------------------------
constexpr int kLutRecs = 1024;
constexpr float kLutScale = 0.5f * (kLutRecs - 2);                    // 511
constexpr float kLutY = 0x1p-22f * kLutScale;
constexpr float kLutMagic = 2.0f + 0x1p-22f * (1.0f + kLutScale);     // 2 + 512 * 2^-22
constexpr double kLutSlack = 0x1p-20;
constexpr int kPairs = 18;                 // pair i < 17: {T[i], T[i + 1]}; pair 17: NaN
constexpr int kNaNPair = 17;

// Group scales outside [2^-30, 2^30] take the exact fallback (no fp32 over/underflow there).
constexpr float kFastScaleMin = 0x1p-30f;
constexpr float kFastScaleMax = 0x1p30f;

// Index of the calling wave in its workgroup, as a wave-uniform (scalar) value: row indices and
// row base addresses derived from it stay in scalar registers.
__device__ __forceinline__ int wave_index() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
}

// The threads that run one kernel body together, here the whole workgroup: tid() is the thread's
// index in the group, wave() the wave's (wave-uniform), sync() the group's barrier. The bodies take
// it as a parameter rather than reading threadIdx and calling __syncthreads themselves.
struct WholeBlock {
  __device__ __forceinline__ int tid() const { return (int)threadIdx.x; }
  __device__ __forceinline__ int wave() const {
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  }
  __device__ __forceinline__ void sync() const { __syncthreads(); }
};

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// Round a finite fp32 value to bf16, ties to even. Truncating 16 bits rounds down in magnitude; adding
// 0x7fff rounds up every remainder above one half, and adding the kept least-significant bit as
// well rounds an exact half up only when the kept part is odd. A carry out of the fraction moves
// into the exponent, which is the correct next binade (or infinity past the largest finite value).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  uint32_t b = __float_as_uint(x);
  return (b + 0x7fffu + ((b >> 16) & 1u)) >> 16;
}

// Butterfly reductions over aligned blocks of `lanes` lanes (a power of two <= 64). Within a row
// of 16 lanes they use DPP: quad_perm [1,0,3,2] and [2,3,0,1] exchange partners at distance 1 and 2,
// row_half_mirror and row_mirror bring in the other quad and the other half-row, whose lanes by then
// all hold the same partial. Larger blocks finish with cross-row shuffles. Every lane of a block
// performs the same additions on the same operands (addition commutes), so all lanes end with
// bitwise identical totals.
constexpr int kDppQuadXor1 = 0xB1;
constexpr int kDppQuadXor2 = 0x4E;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  // every control used here reads a lane of the same 16-lane row, so no lane keeps an old value:
  // mov_dpp needs no initialised destination
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)b, CTRL, 0xF, 0xF, true);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF,
                                                         true);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// LANES > 0: block size known at compile time; LANES == 0: use the runtime value `lanes`.
template <int LANES>
__device__ __forceinline__ uint32_t block_max_u32_t(uint32_t v, int lanes) {
  if (LANES > 0) lanes = LANES;
  if (lanes >= 2) v = max(v, dpp_u32<kDppQuadXor1>(v));
  if (lanes >= 4) v = max(v, dpp_u32<kDppQuadXor2>(v));
  if (lanes >= 8) v = max(v, dpp_u32<kDppRowHalfMirror>(v));
  if (lanes >= 16) v = max(v, dpp_u32<kDppRowMirror>(v));
  if (lanes >= 32) v = max(v, (uint32_t)__shfl_xor((int)v, 16));
  if (lanes >= 64) v = max(v, (uint32_t)__shfl_xor((int)v, 32));
  return v;
}
template <int LANES>
__device__ __forceinline__ double block_sum_f64_t(double v, int lanes) {
  if (LANES > 0) lanes = LANES;
  if (lanes >= 2) v += dpp_f64<kDppQuadXor1>(v);
  if (lanes >= 4) v += dpp_f64<kDppQuadXor2>(v);
  if (lanes >= 8) v += dpp_f64<kDppRowHalfMirror>(v);
  if (lanes >= 16) v += dpp_f64<kDppRowMirror>(v);
  if (lanes >= 32) v += __shfl_xor(v, 16);
  if (lanes >= 64) v += __shfl_xor(v, 32);
  return v;
}

__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, int lanes) {
  if (lanes >= 2) v = max(v, dpp_u32<kDppQuadXor1>(v));
  if (lanes >= 4) v = max(v, dpp_u32<kDppQuadXor2>(v));
  if (lanes >= 8) v = max(v, dpp_u32<kDppRowHalfMirror>(v));
  if (lanes >= 16) v = max(v, dpp_u32<kDppRowMirror>(v));
  if (lanes >= 32) v = max(v, (uint32_t)__shfl_xor((int)v, 16));
  if (lanes >= 64) v = max(v, (uint32_t)__shfl_xor((int)v, 32));
  return v;
}
__device__ __forceinline__ double block_sum_f64(double v, int lanes) {
  if (lanes >= 2) v += dpp_f64<kDppQuadXor1>(v);
  if (lanes >= 4) v += dpp_f64<kDppQuadXor2>(v);
  if (lanes >= 8) v += dpp_f64<kDppRowHalfMirror>(v);
  if (lanes >= 16) v += dpp_f64<kDppRowMirror>(v);
  if (lanes >= 32) v += __shfl_xor(v, 16);
  if (lanes >= 64) v += __shfl_xor(v, 32);
  return v;
}

// Contiguous share of `total` tasks for workgroup b of G: [task_lo(b), task_lo(b + 1)).
__host__ __device__ __forceinline__ int64_t task_lo(int64_t b, int64_t total, int64_t G) {
  return (b * total) / G;
}

// Largest |w| of the 8 bf16 of one lane, as the bf16 magnitude bit pattern (order-preserving).
__device__ __forceinline__ uint32_t lane_absmax_bits(const uint4& v) {
  uint32_t a = max(v.x & 0x7fffu, (v.x >> 16) & 0x7fffu);
  uint32_t b = max(v.y & 0x7fffu, (v.y >> 16) & 0x7fffu);
  uint32_t c = max(v.z & 0x7fffu, (v.z >> 16) & 0x7fffu);
  uint32_t d = max(v.w & 0x7fffu, (v.w >> 16) & 0x7fffu);
  return max(max(a, b), max(c, d));
}

// Largest |w| of the 16 bf16 of two 16-byte loads, as the bf16 magnitude bit pattern: sign bits
// cleared, then packed 16-bit maxima.
__device__ __forceinline__ uint32_t lane_absmax16_bits(const uint4& a, const uint4& b) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  const uint32_t m = 0x7fff7fffu;
  const u16x2 x0 = __builtin_bit_cast(u16x2, a.x & m), x1 = __builtin_bit_cast(u16x2, a.y & m);
  const u16x2 x2 = __builtin_bit_cast(u16x2, a.z & m), x3 = __builtin_bit_cast(u16x2, a.w & m);
  const u16x2 x4 = __builtin_bit_cast(u16x2, b.x & m), x5 = __builtin_bit_cast(u16x2, b.y & m);
  const u16x2 x6 = __builtin_bit_cast(u16x2, b.z & m), x7 = __builtin_bit_cast(u16x2, b.w & m);
  const u16x2 y = __builtin_elementwise_max(
      __builtin_elementwise_max(__builtin_elementwise_max(x0, x1), __builtin_elementwise_max(x2, x3)),
      __builtin_elementwise_max(__builtin_elementwise_max(x4, x5), __builtin_elementwise_max(x6, x7)));
  return max((uint32_t)y.x, (uint32_t)y.y);
}

// Largest |w| of 16 fp32 values, as its fp32 bit pattern (non-negative fp32 values order like
// their bit patterns, so lane partials combine with an integer max). Three-input maxima with
// absolute-value operands: about half the instructions of masking and comparing the packed bf16.
__device__ __forceinline__ uint32_t absmax16_f32_bits(const float (&w)[16]) {
  float m[6];
#pragma unroll
  for (int i = 0; i < 5; ++i)
    m[i] = __builtin_fmaxf(__builtin_fmaxf(fabsf(w[3 * i]), fabsf(w[3 * i + 1])),
                           fabsf(w[3 * i + 2]));
  m[5] = fabsf(w[15]);
  const float a = __builtin_fmaxf(__builtin_fmaxf(m[0], m[1]), m[2]);
  const float b = __builtin_fmaxf(__builtin_fmaxf(m[3], m[4]), m[5]);
  return __float_as_uint(__builtin_fmaxf(a, b));
}

__device__ __forceinline__ void unpack8(const uint4& v, float (&w)[8]) {
  w[0] = bf16_lo(v.x); w[1] = bf16_hi(v.x);
  w[2] = bf16_lo(v.y); w[3] = bf16_hi(v.y);
  w[4] = bf16_lo(v.z); w[5] = bf16_hi(v.z);
  w[6] = bf16_lo(v.w); w[7] = bf16_hi(v.w);
}

// ------------------------------------------------------------------------------------------------
// Job descriptors (kernel arguments, by value).
// ------------------------------------------------------------------------------------------------
struct MatrixGeom {
  int64_t R;
  int32_t C;
  int32_t nslab;       // ceil(C / slab width)
  int64_t task_begin;  // first task of this job in the batch-wide numbering
  int64_t ntasks;      // ceil(R / rows per task) * nslab
};

struct AssignJob {
  MatrixGeom geom;
  const uint16_t* W;
  const float* I;
  const float* tables;      // fp32 [2][n]
  uint32_t* codes;          // [R * C / 8] dwords, 8 nibbles each
  uint8_t* sel;             // [R * C / S]
  double* err;              // nullable, [R * C / S][2]
  double* err_total;        // nullable, one fp64: sum of the chosen errors over the matrix
  int32_t wg_lo;            // first workgroup whose task range meets this job (totals only)
  int32_t wg_count;         // number of such workgroups
};

struct AssignBatch {
  AssignJob job[kMaxJobs];
  int32_t njobs;
  int32_t g, S, n;
  int64_t total_tasks;
  int32_t totals;           // 1: every job's err_total is written (partials/counters given)
  int32_t slots;            // largest wg_count of the batch
  double* partials;         // [njobs][slots] per-workgroup sums of the chosen errors
  uint32_t* counters;       // [njobs], zero between calls
};

// Workgroup b of a grid of nb owns tasks [task_lo(b), task_lo(b + 1)). Records in each job which
// workgroups meet its tasks (wg_lo, wg_count) and returns the largest count.
template <class Job>
inline int32_t job_slots(Job* jobs, int njobs, int64_t total_tasks, int64_t nb) {
  auto owner = [&](int64_t t) {
    int64_t lo = 0, hi = nb - 1;
    while (lo < hi) {
      const int64_t mid = (lo + hi + 1) / 2;
      if (task_lo(mid, total_tasks, nb) <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
  };
  int32_t slots = 1;
  for (int i = 0; i < njobs; ++i) {
    const int64_t w0 = owner(jobs[i].geom.task_begin);
    const int64_t w1 = owner(jobs[i].geom.task_begin + jobs[i].geom.ntasks - 1);
    jobs[i].wg_lo = (int32_t)w0;
    jobs[i].wg_count = (int32_t)(w1 - w0 + 1);
    if (jobs[i].wg_count > slots) slots = jobs[i].wg_count;
  }
  return slots;
}

// Largest assign grid; the error-total workspace holds this many partials per matrix.
constexpr int kMaxAssignBlocks = 4096;

struct RefineJob {
  MatrixGeom geom;
  const uint16_t* W;
  const float* I;
  const uint32_t* codes;
  const uint8_t* sel;
  const float* tables_in;
  float* tables_out;
  uint32_t* codes_out;      // fused assign + accumulate only: where the assign step writes
  uint8_t* sel_out;
  double* err_out;          // nullable: error of the incoming assignment under tables_in
  double* err_after;        // with err_out: the same assignment's error under tables_out
  double* w2;               // with err_out: sum I w^2 (output, or input with the W2-known flag)
  int32_t wg_lo;            // first workgroup whose task range meets this job
  int32_t wg_count;         // number of such workgroups
};

// Per-workgroup partial values of a refine: 64 cell sums (num, den of 32 cells), sum I w^2, pad.
constexpr int kPartVals = 66;
// Largest refine grid; the workspace holds this many partials per matrix.
constexpr int64_t kMaxRefineBlocks = 1024;

struct RefineBatch {
  RefineJob job[kMaxJobs];
  int32_t njobs;
  int32_t g, S, n;
  int64_t total_tasks;
  double* partials;         // [njobs][kPartVals][slots]
  uint32_t* counters;       // [njobs], zero between calls
  int32_t nblocks;          // grid size
  int32_t slots;            // largest wg_count of the batch
  int32_t flags;            // bit 0: round to bf16; bit 1: W2 given
  int32_t errs;             // 1: the jobs have err_out
};

// ------------------------------------------------------------------------------------------------
// Host launchers (defined next to their kernels). All return hipSuccess or the launch error.
// ------------------------------------------------------------------------------------------------
int device_cu_count();

// with_err: the per-group error array (kErrFull); b.totals: the per-matrix totals.
hipError_t launch_assign(const AssignBatch& b, bool with_err, hipStream_t stream);
hipError_t launch_refine(RefineBatch& b, hipStream_t stream);
int refine_grid(int64_t total_tasks);
// One launch doing a batched assign and then a batched refine on its codes (selection groups of at
// least 16 weights); same geometry and workspace as the refine launch, same results bit for bit.
hipError_t launch_assign_refine(RefineBatch& b, hipStream_t stream);
// Task geometry of the refine kernel for one matrix (it depends on the selection group size).
MatrixGeom refine_geom(int64_t R, int64_t C, int64_t task_begin, int S);

hipError_t launch_importance(const float* X, int64_t T, int64_t K, int64_t ldx, double* I_acc,
                             float* I_out, double* partials, int nsplit, hipStream_t stream);
int importance_splits(int64_t T, int64_t K);

size_t init_workspace_bytes(int count, const int64_t* R, const int64_t* C);
hipError_t launch_init(int count, const uint16_t* const* W, const int64_t* R, const int64_t* C,
                       int g, int n, float* const* tables, void* ws, hipStream_t stream);

hipError_t launch_pack(int count, const uint16_t* const* W, const int64_t* R, const int64_t* C,
                       int g, int S, int n, const uint8_t* const* sel, const float* const* tables,
                       uint16_t* const* scales, uint8_t* const* bitmap,
                       uint16_t* const* tables_bf16, hipStream_t stream);
// Codes one per byte ([R * C], low nibble) into two per byte ([R * C / 2]).
hipError_t launch_pack_codes(const uint8_t* codes_u8, uint8_t* codes_out, int64_t R, int64_t C,
                             hipStream_t stream);
hipError_t launch_dequant(int count, const uint8_t* const* codes, const uint16_t* const* scales,
                          const uint8_t* const* bitmap, const uint16_t* const* tables_bf16,
                          const int64_t* R, const int64_t* C, int g, int S, int n,
                          uint16_t* const* W_hat, hipStream_t stream);
// Decode GEMV over up to kMaxJobs packed matrices that share g, S, n and the batch size B.
struct GemvJob {
  const uint8_t* codes;      // [R, C / 2]
  const uint16_t* scales;    // [R, C / g]
  const uint8_t* bitmap;     // S < g, else null
  const uint16_t* tables;    // bf16 [2][n]
  const uint16_t* x;         // bf16 [B, C]
  float* y;                  // [B, R]
  int64_t R, C;
  int64_t task_begin;        // first workgroup task of this matrix
  int split;                 // waves per row block (1, 2 or 4), from the slab count
};
struct GemvBatch {
  GemvJob job[kMaxJobs];
  int njobs, B, g, S, n;
  int64_t total_tasks;
};
int gemv_split(int64_t C);
int64_t gemv_tasks(int64_t R, int64_t C);
hipError_t launch_gemv(const GemvBatch& b, hipStream_t stream);

hipError_t launch_awq_prescale(const uint16_t* W, int64_t R, int64_t C, const float* a,
                               const float* I, uint16_t* W_scaled, float* I_scaled,
                               hipStream_t stream);

inline MatrixGeom make_geom(int64_t R, int64_t C, int64_t task_begin, int slab = kSlab,
                            int rows_per_task = kRowsPerTask) {
  MatrixGeom m;
  m.R = R;
  m.C = (int32_t)C;
  m.nslab = (int32_t)((C + slab - 1) / slab);
  m.task_begin = task_begin;
  m.ntasks = ((R + rows_per_task - 1) / rows_per_task) * (int64_t)m.nslab;
  return m;
}

}  // namespace aaac
