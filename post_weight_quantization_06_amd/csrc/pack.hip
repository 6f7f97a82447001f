// Stored format (AAAC summary §2 mechanism 3, §4) and dequantization (§1).
//
// pack:    bf16 group scales with the selector in the sign bit (S == g) or a separate LSB-first
//          bitmap of selectors (S < g), and the bf16 tables. The codes are written by assign.
// dequant: W_hat = bf16(|s| * T~_sel[q]); the product of two bf16 values is exact in fp32 whenever
//          it is a normal number, so there is a single rounding (ties to even); products below
//          2^-126 are formed in fp64 and rounded once from there.
#include "common.h"

namespace aaac {

// Up to kMaxJobs matrices that share g, S and n; a single call is a batch of one.
struct PackJob {
  const uint16_t* W;
  MatrixGeom geom;              // task numbering shared by the batch (32 rows x 512 columns)
  const uint8_t* sel;
  uint16_t* scales;
  uint8_t* bitmap;              // S < g, else null
  const float* tables;
  uint16_t* tables_bf16;
  int64_t byte_begin;           // first bitmap byte (or table item) of this job, batch-wide
  int64_t nbytes;               // bitmap bytes of this job (0 when S == g)
};

struct PackBatch {
  PackJob job[kMaxJobs];
  int njobs, g, S, n;
  int64_t total_tasks, total_items;
};

constexpr int kDequantSteps = 4;
constexpr int64_t kDequantTaskVecs = (int64_t)kBlock * kDequantSteps;

struct DequantJob {
  const uint32_t* codes;        // one word per 8 weights
  const uint16_t* scales;
  const uint8_t* bitmap;        // S < g, else null
  const uint16_t* tables_bf16;
  uint4* out;                   // 8 bf16 per vector
  int64_t task_begin;           // first task (kDequantTaskVecs vectors) of this job, batch-wide
  int64_t nvec;
};

struct DequantBatch {
  DequantJob job[kMaxJobs];
  int njobs, g, S, n;
  int64_t total_tasks;
};

// The scale word of every scale group: lane mapping of the 8-weight assign (a lane holds 8
// consecutive weights of a row, a group spans g / 8 lanes). One workgroup per task; the rows of a
// task are all loaded first (unconditional loads at clamped in-bounds addresses), so a wave keeps
// eight rows in flight. With the selector in the sign bit (S == g) the first workgroup of each
// matrix also converts its tables; with a bitmap the bits kernel does.
__global__ __launch_bounds__(kBlock) void pack_scales_kernel(PackBatch b) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave, g8 = b.g / kPerLane;
  const int log2g = 31 - __builtin_clz((unsigned)b.g), log2S = 31 - __builtin_clz((unsigned)b.S);
  for (int64_t task = blockIdx.x; task < b.total_tasks; task += gridDim.x) {
    int j = 0;
    while (j + 1 < b.njobs && task >= b.job[j + 1].geom.task_begin) ++j;
    const PackJob& jb = b.job[j];
    if (jb.bitmap == nullptr && task == jb.geom.task_begin && tid < 2 * b.n)
      jb.tables_bf16[tid] = (uint16_t)f32_to_bf16_rne(jb.tables[tid]);
    const int64_t R = jb.geom.R, C = jb.geom.C;
    const int64_t local = task - jb.geom.task_begin;
    const int64_t rb = local / jb.geom.nslab;
    const int slab = (int)(local - rb * jb.geom.nslab);
    const int c0 = slab * kSlab + lane * kPerLane;
    const bool active = c0 < C;
    const int cl = active ? c0 : 0;
    const int64_t r0 = rb * kRowsPerTask + wave;
    uint4 v[kRowsPerWave];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      int64_t r = r0 + (int64_t)kWavesPerBlock * i;
      r = r < R ? r : R - 1;
      v[i] = *reinterpret_cast<const uint4*>(jb.W + r * C + cl);
    }
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      const int64_t r = r0 + (int64_t)kWavesPerBlock * i;
      if (r >= R) break;                              // the same for the whole wave
      const uint32_t amax = block_max_u32(lane_absmax_bits(v[i]), g8);
      if (active && ((c0 >> 3) & (g8 - 1)) == 0) {
        const int64_t base = r * C + c0;
        uint32_t word = amax;
        if (b.S == b.g) word |= (jb.sel[base >> log2S] ? 1u : 0u) << 15;
        jb.scales[base >> log2g] = (uint16_t)word;
      }
    }
  }
}

// S < g: the selector bitmap, one byte (8 selection groups) per thread over the batch's bytes,
// and the tables (the first 2n items of each matrix).
__global__ __launch_bounds__(kBlock) void pack_bits_kernel(PackBatch b) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (i >= b.total_items) return;
  int j = 0;
  while (j + 1 < b.njobs && i >= b.job[j + 1].byte_begin) ++j;
  const PackJob& jb = b.job[j];
  const int64_t local = i - jb.byte_begin;
  if (local < 2 * b.n) jb.tables_bf16[local] = (uint16_t)f32_to_bf16_rne(jb.tables[local]);
  if (local >= jb.nbytes) return;
  const int64_t ngroups = jb.geom.R * jb.geom.C / b.S;
  uint32_t bits = 0;
  for (int k = 0; k < 8; ++k) {
    const int64_t h = local * 8 + k;
    if (h < ngroups && jb.sel[h]) bits |= 1u << k;
  }
  jb.bitmap[local] = (uint8_t)bits;
}

// Two finite fp32 values rounded to bf16 (ties to even) and packed, lo in the low half: one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// fp64 value -> bf16 bits, ties to even, by exact scaling to the binade's quantum.
__device__ __forceinline__ uint32_t f64_to_bf16_bits(double x) {
  if (x == 0.0) return (__double_as_longlong(x) >> 48) & 0x8000u;
  const double ax = fabs(x);
  const int e = ax < 0x1p-126 ? -126 : ilogb(ax);
  const double q = ldexp(1.0, e - 7);
  const double r = rint(ax / q) * q;
  uint32_t bits = r >= 0x1p128 ? 0x7f80u : (__float_as_uint((float)r) >> 16);
  if (x < 0.0) bits |= 0x8000u;
  return bits;
}

// A thread dequantizes 8 weights (one code word) per step, four steps with their loads in flight;
// a workgroup takes tasks of 1024 vectors of one matrix, so the matrix's fields are uniform and
// every step reads 256 consecutive code words and writes 4 KB in one piece.
__global__ __launch_bounds__(kBlock) void dequant_kernel(DequantBatch b) {
  __shared__ float tab[2][16];
  const int n = b.n;
  const int log2g = 31 - __builtin_clz((unsigned)b.g), log2S = 31 - __builtin_clz((unsigned)b.S);
  int cur = -1;
  for (int64_t task = blockIdx.x; task < b.total_tasks; task += gridDim.x) {
    int j = 0;
    while (j + 1 < b.njobs && task >= b.job[j + 1].task_begin) ++j;
    const DequantJob& jb = b.job[j];
    if (j != cur) {
      __syncthreads();
      if (threadIdx.x < 2 * n)
        tab[threadIdx.x / n][threadIdx.x % n] =
            __uint_as_float((uint32_t)jb.tables_bf16[threadIdx.x] << 16);
      __syncthreads();
      cur = j;
    }
    const int64_t nvec = jb.nvec;
    const int64_t i0 = (task - jb.task_begin) * kDequantTaskVecs + threadIdx.x;
    uint32_t cw[kDequantSteps], word[kDequantSteps], sg[kDequantSteps];
#pragma unroll
    for (int u = 0; u < kDequantSteps; ++u) {
      int64_t i = i0 + (int64_t)u * kBlock;
      i = i < nvec ? i : nvec - 1;                    // in bounds; the result is not stored
      const int64_t base = i * 8;
      cw[u] = jb.codes[i];
      word[u] = jb.scales[base >> log2g];
      if (jb.bitmap == nullptr) {
        sg[u] = word[u] >> 15;
      } else {
        const int64_t h = base >> log2S;
        sg[u] = (jb.bitmap[h >> 3] >> (h & 7)) & 1u;
      }
    }
#pragma unroll
    for (int u = 0; u < kDequantSteps; ++u) {
      const int64_t i = i0 + (int64_t)u * kBlock;
      if (i >= nvec) break;
      const float s = __uint_as_float((word[u] & 0x7fffu) << 16);
      float t[8], p[8];
      bool tiny = false;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t q = (cw[u] >> (4 * k)) & 15u;
        t[k] = tab[sg[u]][q < (uint32_t)n ? q : 0];
        p[k] = s * t[k];
        // exact in fp32 unless the product is a nonzero subnormal (or underflows to zero)
        tiny = tiny || (fabsf(p[k]) < 0x1p-126f && s != 0.0f && t[k] != 0.0f);
      }
      // pairs of exact products rounded to bf16 (ties to even) by the conversion instruction
      uint32_t o[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) o[k] = pack_bf16x2(p[2 * k], p[2 * k + 1]);
      if (tiny) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          if (fabsf(p[k]) < 0x1p-126f && s != 0.0f && t[k] != 0.0f) {
            const uint32_t bits = f64_to_bf16_bits((double)s * (double)t[k]);
            const int sh = 16 * (k & 1);
            o[k >> 1] = (o[k >> 1] & ~(0xffffu << sh)) | (bits << sh);
          }
        }
      }
      jb.out[i] = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

hipError_t launch_pack(int count, const uint16_t* const* W, const int64_t* R, const int64_t* C,
                       int g, int S, int n, const uint8_t* const* sel, const float* const* tables,
                       uint16_t* const* scales, uint8_t* const* bitmap,
                       uint16_t* const* tables_bf16, hipStream_t stream) {
  PackBatch b{};
  b.njobs = count;
  b.g = g;
  b.S = S;
  b.n = n;
  const bool bits = S < g;
  int64_t tb = 0, items = 0;
  for (int i = 0; i < count; ++i) {
    PackJob& j = b.job[i];
    j.W = W[i];
    j.geom = make_geom(R[i], C[i], tb);
    tb += j.geom.ntasks;
    j.sel = sel[i];
    j.scales = scales[i];
    j.bitmap = bits ? bitmap[i] : nullptr;
    j.tables = tables[i];
    j.tables_bf16 = tables_bf16[i];
    j.nbytes = bits ? (R[i] * C[i] / S + 7) / 8 : 0;
    j.byte_begin = items;
    items += j.nbytes > 2 * n ? j.nbytes : 2 * n;
  }
  b.total_tasks = tb;
  b.total_items = items;
  // one task per workgroup (up to 2^20, then a grid-stride loop): the dispatcher balances the
  // tail, where a grid of a few workgroups per CU looping over the tasks left its last round
  // partly empty
  const int64_t want = 1 << 20;
  const int grid = (int)(tb < want ? tb : want);
  hipLaunchKernelGGL(pack_scales_kernel, dim3(grid > 0 ? grid : 1), dim3(kBlock), 0, stream, b);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !bits) return e;
  hipLaunchKernelGGL(pack_bits_kernel, dim3((unsigned)((items + kBlock - 1) / kBlock)),
                     dim3(kBlock), 0, stream, b);
  return hipGetLastError();
}

// Codes given one per byte (low nibble; the high nibble is ignored) packed two per byte, the even
// column in the low nibble: 8 codes in, one 32-bit word out per thread.
__global__ __launch_bounds__(kBlock) void pack_codes_kernel(const uint2* __restrict__ in,
                                                            uint32_t* __restrict__ out,
                                                            int64_t items) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < items; i += stride) {
    const uint2 v = in[i];
    // bytes b0..b3 of v.x hold codes 0..3; keep each low nibble and pair them
    const uint32_t x = v.x & 0x0F0F0F0Fu, y = v.y & 0x0F0F0F0Fu;
    const uint32_t px = (x | (x >> 4)) & 0x00FF00FFu;    // bytes 0 and 2: codes 0|1, 2|3
    const uint32_t py = (y | (y >> 4)) & 0x00FF00FFu;
    out[i] = __builtin_amdgcn_perm(py, px, 0x06040200u);
  }
}

hipError_t launch_pack_codes(const uint8_t* codes_u8, uint8_t* codes_out, int64_t R, int64_t C,
                             hipStream_t stream) {
  const int64_t items = R * C / 8;
  if (items <= 0) return hipSuccess;
  const int64_t cap = (int64_t)device_cu_count() * 8;
  int64_t grid = (items + kBlock - 1) / kBlock;
  if (grid > cap) grid = cap;
  hipLaunchKernelGGL(pack_codes_kernel, dim3((unsigned)grid), dim3(kBlock), 0, stream,
                     reinterpret_cast<const uint2*>(codes_u8),
                     reinterpret_cast<uint32_t*>(codes_out), items);
  return hipGetLastError();
}

hipError_t launch_dequant(int count, const uint8_t* const* codes, const uint16_t* const* scales,
                          const uint8_t* const* bitmap, const uint16_t* const* tables_bf16,
                          const int64_t* R, const int64_t* C, int g, int S, int n,
                          uint16_t* const* W_hat, hipStream_t stream) {
  DequantBatch b{};
  b.njobs = count;
  b.g = g;
  b.S = S;
  b.n = n;
  int64_t tasks = 0;
  for (int i = 0; i < count; ++i) {
    DequantJob& j = b.job[i];
    j.codes = reinterpret_cast<const uint32_t*>(codes[i]);
    j.scales = scales[i];
    j.bitmap = S < g ? bitmap[i] : nullptr;
    j.tables_bf16 = tables_bf16[i];
    j.out = reinterpret_cast<uint4*>(W_hat[i]);
    j.task_begin = tasks;
    j.nvec = R[i] * C[i] / 8;
    tasks += (j.nvec + kDequantTaskVecs - 1) / kDequantTaskVecs;
  }
  b.total_tasks = tasks;
  // up to 8 workgroups per CU walking the tasks: a workgroup per task paid its table load and
  // barriers for every 1024 vectors
  const int64_t cap = (int64_t)device_cu_count() * 8;
  int64_t grid = tasks < cap ? tasks : cap;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)grid), dim3(kBlock), 0, stream, b);
  return hipGetLastError();
}

}  // namespace aaac
