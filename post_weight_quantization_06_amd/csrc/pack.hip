// Stored format (AAAC summary §2 mechanism 3, §4) and dequantization (§1).
//
// pack:    bf16 group scales with the selector in the sign bit (S == g) or a separate LSB-first
//          bitmap of selectors (S < g), and the bf16 tables. The codes are written by assign.
// dequant: W_hat = bf16(|s| * T~_sel[q]); the product of two bf16 values is exact in fp32 whenever
//          it is a normal number, so there is a single rounding (ties to even); products below
//          2^-126 are formed in fp64 and rounded once from there.
#include "common.h"

namespace aaac {

// The scale word of every scale group: lane mapping of the 8-weight assign (a lane holds 8
// consecutive weights of a row, a group spans g / 8 lanes). The rows of a task are all loaded first
// (unconditional loads at clamped in-bounds addresses), so a wave keeps eight rows in flight.
__global__ __launch_bounds__(kBlock) void pack_scales_kernel(const uint16_t* __restrict__ W,
                                                             MatrixGeom geom, int g, int S,
                                                             const uint8_t* __restrict__ sel,
                                                             uint16_t* __restrict__ scales,
                                                             const float* __restrict__ tables,
                                                             int n,
                                                             uint16_t* __restrict__ tables_bf16) {
  const int tid = threadIdx.x;
  // the tables, when no bitmap kernel follows to convert them
  if (tables_bf16 != nullptr && blockIdx.x == 0 && tid < 2 * n)
    tables_bf16[tid] = (uint16_t)f32_to_bf16_rne(tables[tid]);
  const int lane = tid & (kWave - 1), wave = tid / kWave, g8 = g / kPerLane;
  const int log2g = 31 - __builtin_clz((unsigned)g), log2S = 31 - __builtin_clz((unsigned)S);
  const int64_t R = geom.R, C = geom.C;
  for (int64_t task = blockIdx.x; task < geom.ntasks; task += gridDim.x) {
    const int64_t rb = task / geom.nslab;
    const int slab = (int)(task - rb * geom.nslab);
    const int c0 = slab * kSlab + lane * kPerLane;
    const bool active = c0 < C;
    const int cl = active ? c0 : 0;
    const int64_t r0 = rb * kRowsPerTask + wave;
    uint4 v[kRowsPerWave];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      int64_t r = r0 + (int64_t)kWavesPerBlock * i;
      r = r < R ? r : R - 1;
      v[i] = *reinterpret_cast<const uint4*>(W + r * C + cl);
    }
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      const int64_t r = r0 + (int64_t)kWavesPerBlock * i;
      if (r >= R) break;                              // the same for the whole wave
      const uint32_t amax = block_max_u32(lane_absmax_bits(v[i]), g8);
      if (active && ((c0 >> 3) & (g8 - 1)) == 0) {
        const int64_t base = r * C + c0;
        uint32_t word = amax;
        if (S == g) word |= (sel[base >> log2S] ? 1u : 0u) << 15;
        scales[base >> log2g] = (uint16_t)word;
      }
    }
  }
}

__global__ __launch_bounds__(kBlock) void pack_bits_kernel(const uint8_t* __restrict__ sel,
                                                           int64_t ngroups,
                                                           uint8_t* __restrict__ bitmap,
                                                           const float* __restrict__ tables,
                                                           int n, uint16_t* __restrict__ tables_bf16) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (i < 2 * n) tables_bf16[i] = (uint16_t)f32_to_bf16_rne(tables[i]);
  if (bitmap == nullptr) return;
  const int64_t nbytes = (ngroups + 7) / 8;
  if (i >= nbytes) return;
  uint32_t b = 0;
  for (int k = 0; k < 8; ++k) {
    const int64_t h = i * 8 + k;
    if (h < ngroups && sel[h]) b |= 1u << k;
  }
  bitmap[i] = (uint8_t)b;
}

hipError_t launch_pack(const uint16_t* W, int64_t R, int64_t C, int g, int S, int n,
                       const uint8_t* sel, const float* tables, uint16_t* scales, uint8_t* bitmap,
                       uint16_t* tables_bf16, hipStream_t stream) {
  const MatrixGeom geom = make_geom(R, C, 0);
  // one task per workgroup (up to 2^20, then a grid-stride loop): the dispatcher balances the
  // tail, where a grid of a few workgroups per CU looping over the tasks left its last round
  // partly empty
  const int64_t want = 1 << 20;
  const int grid = (int)(geom.ntasks < want ? geom.ntasks : want);
  // with the selection bit in the scale's sign there is no bitmap, and the scales kernel converts
  // the tables itself: one launch instead of two
  const bool bits = S < g;
  hipLaunchKernelGGL(pack_scales_kernel, dim3(grid), dim3(kBlock), 0, stream, W, geom, g, S, sel,
                     scales, tables, n, bits ? nullptr : tables_bf16);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !bits) return e;
  const int64_t ngroups = R * C / S;
  int64_t items = (ngroups + 7) / 8;
  if (items < 2 * n) items = 2 * n;
  hipLaunchKernelGGL(pack_bits_kernel, dim3((unsigned)((items + kBlock - 1) / kBlock)),
                     dim3(kBlock), 0, stream, sel, ngroups, bitmap, tables, n, tables_bf16);
  return hipGetLastError();
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

// A thread dequantizes 8 weights (one code word) per step, four steps with their loads in flight.
__global__ __launch_bounds__(kBlock) void dequant_kernel(const uint32_t* __restrict__ codes,
                                                         const uint16_t* __restrict__ scales,
                                                         const uint8_t* __restrict__ bitmap,
                                                         const uint16_t* __restrict__ tables_bf16,
                                                         int64_t R, int64_t C, int g, int S, int n,
                                                         uint4* __restrict__ out) {
  __shared__ float tab[2][16];
  if (threadIdx.x < 2 * n)
    tab[threadIdx.x / n][threadIdx.x % n] = __uint_as_float((uint32_t)tables_bf16[threadIdx.x] << 16);
  __syncthreads();
  const int log2g = 31 - __builtin_clz((unsigned)g), log2S = 31 - __builtin_clz((unsigned)S);
  const int64_t nvec = R * C / 8;
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  constexpr int kSteps = 4;
  for (int64_t i0 = (int64_t)blockIdx.x * kBlock + threadIdx.x; i0 < nvec; i0 += kSteps * stride) {
    uint32_t cw[kSteps], word[kSteps], sg[kSteps];
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
      int64_t i = i0 + u * stride;
      i = i < nvec ? i : nvec - 1;                    // in bounds; the result is not stored
      const int64_t base = i * 8;
      cw[u] = codes[i];
      word[u] = scales[base >> log2g];
      if (bitmap == nullptr) {
        sg[u] = word[u] >> 15;
      } else {
        const int64_t h = base >> log2S;
        sg[u] = (bitmap[h >> 3] >> (h & 7)) & 1u;
      }
    }
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
      const int64_t i = i0 + u * stride;
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
            const uint32_t b = f64_to_bf16_bits((double)s * (double)t[k]);
            const int sh = 16 * (k & 1);
            o[k >> 1] = (o[k >> 1] & ~(0xffffu << sh)) | (b << sh);
          }
        }
      }
      out[i] = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

hipError_t launch_dequant(const uint8_t* codes, const uint16_t* scales, const uint8_t* bitmap,
                          const uint16_t* tables_bf16, int64_t R, int64_t C, int g, int S, int n,
                          uint16_t* W_hat, hipStream_t stream) {
  const int64_t nvec = R * C / 8;
  int64_t grid = (nvec + kBlock - 1) / kBlock;
  const int64_t cap = (int64_t)device_cu_count() * 8;
  if (grid > cap) grid = cap;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)grid), dim3(kBlock), 0, stream,
                     reinterpret_cast<const uint32_t*>(codes), scales, S < g ? bitmap : nullptr,
                     tables_bf16, R, C, g, S, n, reinterpret_cast<uint4*>(W_hat));
  return hipGetLastError();
}

}  // namespace aaac
