// Assign step (AAAC summary §2 mechanisms 2 and 4) and the nearest-entry lookup structure it uses.
//
// For every weight w of a scale group with scale s = max|w| and each table c, the nearest entry
// q_c minimizes |u - T_c[j]| with u = w / s, ties to the lower index. Because s > 0 this is the
// same as minimizing |w - s T_c[j]|, and the kernel decides it on r = fma(-s, T, w), the exactly
// rounded residual: when the rounded magnitudes differ, the exact ones differ the same way, and
// when they are equal the two squared distances agree to 2^-22 relative. Candidates come from a
// 1024-record table indexed by an approximate u, built so that each record lists every entry that
// can be nearest anywhere in (a slightly widened copy of) its interval; a record that would need
// more than two candidates routes its group to an exact full scan.
//
// Per selection group the kernel forms D = E_1 - E_0 = sum I_k (m_1^2 - m_0^2) with m_c the chosen
// residual magnitude: fp32 over four weights, then fp64. The selection is D < 0 (ties keep T0).
// Its rounding error is below 8 * 2^-24 (E_0 + E_1), so a selection can only differ from the exact
// one when |E_1 - E_0| < 1e-6 max(E_0, E_1).
#include "common.h"

namespace aaac {

// ------------------------------------------------------------------------------------------------
// Lookup structure: one workgroup per table pair.
// ------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void lut_build_kernel(LutBatch b) {
  const float* T = b.tables[blockIdx.x];
  uint8_t* out = b.lut[blockIdx.x];
  const int n = b.n;
  __shared__ float sv[2][16];
  __shared__ int six[2][16];
  __shared__ double smid[2][16];
  __shared__ int sm[2];
  const int tid = threadIdx.x;
  if (tid < 2) {
    const int c = tid;
    float v[16];
    int ix[16];
    bool finite = true;
    for (int j = 0; j < n; ++j) {
      v[j] = T[c * n + j];
      ix[j] = j;
      finite = finite && isfinite(v[j]);
    }
    // insertion sort by (value, index); equal values keep index order
    for (int i = 1; i < n; ++i) {
      float x = v[i];
      int xi = ix[i];
      int k = i - 1;
      while (k >= 0 && v[k] > x) {
        v[k + 1] = v[k];
        ix[k + 1] = ix[k];
        --k;
      }
      v[k + 1] = x;
      ix[k + 1] = xi;
    }
    // distinct values, each with the lowest index that holds it (the argmin tie rule)
    int m = 0;
    for (int i = 0; i < n; ++i) {
      if (m == 0 || v[i] != sv[c][m - 1]) {
        sv[c][m] = v[i];
        six[c][m] = ix[i];
        ++m;
      }
    }
    for (int i = 0; i + 1 < m; ++i) smid[c][i] = 0.5 * ((double)sv[c][i] + (double)sv[c][i + 1]);
    sm[c] = finite ? m : 0;
  }
  __syncthreads();
  constexpr uint32_t kNaNBits = 0x7fc00000u;
  for (int rho = tid; rho < kLutRecs; rho += kBlock) {
    const double lo = (32.0 * rho - 32.5) / (16.0 * kLutBuckets) - 1.0 - kLutSlack;
    const double hi = (32.0 * rho - 0.5) / (16.0 * kLutBuckets) - 1.0 + kLutSlack;
    uint32_t bits[4];
    uint32_t code = 0;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int m = sm[c];
      int below = 0, inside = 0;
      for (int i = 0; i + 1 < m; ++i) {
        const double M = smid[c][i];
        below += (M < lo) ? 1 : 0;
        inside += (M >= lo && M <= hi) ? 1 : 0;
      }
      // indices clamped so that every read stays inside the arrays whatever the branch
      const int j0 = below < 15 ? below : 15;
      const int j1 = below + 1 < 15 ? below + 1 : 15;
      const bool single = m > 0 && inside == 0;
      const bool pair = m > 0 && inside == 1 && six[c][j1] == six[c][j0] + 1;
      const uint32_t a = __float_as_uint(sv[c][j0]);
      const uint32_t b = __float_as_uint(sv[c][j1]);
      bits[2 * c] = (single || pair) ? a : kNaNBits;
      bits[2 * c + 1] = single ? a : (pair ? b : kNaNBits);
      code |= (single || pair) ? ((uint32_t)six[c][j0] << (4 * c)) : 0u;
    }
    uint4* rec = reinterpret_cast<uint4*>(out + (size_t)rho * kLutRecBytes);
    rec[0] = make_uint4(bits[0], bits[1], bits[2], bits[3]);
    rec[1] = make_uint4(code, 0u, 0u, 0u);
  }
}

hipError_t launch_lut_build(const LutBatch& b, int njobs, hipStream_t stream) {
  hipLaunchKernelGGL(lut_build_kernel, dim3(njobs), dim3(kBlock), 0, stream, b);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------
// Assign kernel.
// ------------------------------------------------------------------------------------------------
struct RowOut {
  double D;         // E_1 - E_0 of the lane's selection group (after the butterfly)
  double E0, E1;    // only with err output
  uint32_t P, Q;    // code bytes (q0 | q1 << 4) of weights 0-3 and 4-7
};

// Exact fallback for one lane: full scan of both tables on scaled operands (w and s multiplied by a
// power of two that brings s into [1, 4), so no residual under- or overflows).
template <bool WITH_ERR>
__device__ __forceinline__ void slow_lane(const float (&w)[8], uint32_t amax, const float (&Ik)[8],
                                          const float (*tab)[16], int n, RowOut& o) {
  const uint32_t E = min(max(amax >> 7, 1u), 253u);
  const float P = __uint_as_float((254u - E) << 23);
  const float sp = __uint_as_float(amax << 16) * P;
  double D = 0.0, E0 = 0.0, E1 = 0.0;
  uint32_t Pw = 0, Qw = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float wp = w[k] * P;
    float best0 = __builtin_inff(), best1 = __builtin_inff();
    uint32_t q0 = 0, q1 = 0;
    for (int j = 0; j < n; ++j) {
      const float r0 = fabsf(__builtin_fmaf(-sp, tab[0][j], wp));
      const float r1 = fabsf(__builtin_fmaf(-sp, tab[1][j], wp));
      if (r0 < best0) { best0 = r0; q0 = j; }
      if (r1 < best1) { best1 = r1; q1 = j; }
    }
    const double b0 = (double)best0 * (double)best0;
    const double b1 = (double)best1 * (double)best1;
    D += (double)Ik[k] * (b1 - b0);
    if (WITH_ERR) {
      E0 += (double)Ik[k] * b0;
      E1 += (double)Ik[k] * b1;
    }
    const uint32_t c = q0 | (q1 << 4);
    if (k < 4) Pw |= c << (8 * k); else Qw |= c << (8 * (k - 4));
  }
  const double inv = 1.0 / ((double)P * (double)P);
  o.D = D;
  o.E0 = E0 * inv;
  o.E1 = E1 * inv;
  o.P = Pw;
  o.Q = Qw;
}

template <bool WITH_ERR>
__device__ __forceinline__ void assign_row(const AssignJob& jb, const uint8_t* __restrict__ lut,
                                           const float (*tab)[16], int n, int g8, int s8, int S,
                                           int64_t r, int c0, bool active, const float (&Ik)[8]) {
  const int64_t base = r * (int64_t)jb.geom.C + c0;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (active) v = *reinterpret_cast<const uint4*>(jb.W + base);
  const uint32_t amax = block_max_u32(lane_absmax_bits(v), g8);
  const float s = __uint_as_float(amax << 16);
  float w[8];
  unpack8(v, w);
  const bool zero = (s == 0.0f);
  const bool fast_scale = zero || (s >= kFastScaleMin && s <= kFastScaleMax);
  const float se = zero ? 1.0f : s;
  const float Y = kLutScale * __builtin_amdgcn_rcpf(se);
  const float nse = -se;

  float acc = 0.0f, a0 = 0.0f, a1 = 0.0f;
  double accd = 0.0, e0d = 0.0, e1d = 0.0;
  uint32_t Pw = 0, Qw = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float t = __builtin_fmaf(w[k], Y, kLutMagic);
    const uint32_t off = __float_as_uint(t) & kLutMask;
    const float4 rec = *reinterpret_cast<const float4*>(lut + off);
    const uint32_t cb = lut[off + 16];
    const float r0a = __builtin_fmaf(nse, rec.x, w[k]);
    const float r0b = __builtin_fmaf(nse, rec.y, w[k]);
    const float r1a = __builtin_fmaf(nse, rec.z, w[k]);
    const float r1b = __builtin_fmaf(nse, rec.w, w[k]);
    const bool d0 = fabsf(r0b) < fabsf(r0a);
    const bool d1 = fabsf(r1b) < fabsf(r1a);
    const float m0 = fminf(fabsf(r0a), fabsf(r0b));
    const float m1 = fminf(fabsf(r1a), fabsf(r1b));
    const float e0 = m0 * m0;
    acc = __builtin_fmaf(Ik[k], __builtin_fmaf(m1, m1, -e0), acc);
    if (WITH_ERR) {
      a0 = __builtin_fmaf(Ik[k], e0, a0);
      a1 = __builtin_fmaf(Ik[k], m1 * m1, a1);
    }
    const uint32_t c = cb + (d0 ? 1u : 0u) + (d1 ? 16u : 0u);
    if (k < 4) Pw |= c << (8 * k); else Qw |= c << (8 * (k - 4));
    if (k == 3 || k == 7) {
      accd += (double)acc;
      acc = 0.0f;
      if (WITH_ERR) {
        e0d += (double)a0;
        e1d += (double)a1;
        a0 = 0.0f;
        a1 = 0.0f;
      }
    }
  }
  RowOut o;
  o.D = block_sum_f64(accd, s8);
  o.E0 = WITH_ERR ? block_sum_f64(e0d, s8) : 0.0;
  o.E1 = WITH_ERR ? block_sum_f64(e1d, s8) : 0.0;
  o.P = Pw;
  o.Q = Qw;
  if (zero) {
    o.D = 0.0;
    o.E0 = 0.0;
    o.E1 = 0.0;
  }
  const bool bad = active && (!fast_scale || !(fabs(o.D) < __builtin_inf()));
  if (__any(bad)) {
    RowOut so;
    slow_lane<WITH_ERR>(w, amax, Ik, tab, n, so);
    so.D = block_sum_f64(so.D, s8);
    if (WITH_ERR) {
      so.E0 = block_sum_f64(so.E0, s8);
      so.E1 = block_sum_f64(so.E1, s8);
    }
    if (bad) o = so;
  }
  const uint32_t sel = (o.D < 0.0) ? 1u : 0u;
  const uint32_t sh = sel ? 4u : 0u;
  uint32_t p = (o.P >> sh) & 0x0F0F0F0Fu;
  uint32_t q = (o.Q >> sh) & 0x0F0F0F0Fu;
  p |= p >> 4;
  q |= q >> 4;
  const uint32_t packed = __builtin_amdgcn_perm(q, p, 0x06040200u);
  if (active) {
    jb.codes[base >> 3] = packed;
    if (((c0 >> 3) & (s8 - 1)) == 0) {
      const int64_t h = base / S;
      jb.sel[h] = (uint8_t)sel;
      if (WITH_ERR) {
        jb.err[2 * h] = o.E0;
        jb.err[2 * h + 1] = o.E1;
      }
    }
  }
}

template <bool WITH_ERR>
__global__ __launch_bounds__(kBlock) void assign_kernel(AssignBatch b) {
  __shared__ __align__(16) uint8_t lut[kLutBytes];
  __shared__ float tab[2][16];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int g8 = b.g / kPerLane, s8 = b.S / kPerLane, n = b.n, S = b.S;
  int cur = -1;
  for (int64_t task = blockIdx.x; task < b.total_tasks; task += gridDim.x) {
    int j = 0;
    while (j + 1 < b.njobs && task >= b.job[j + 1].geom.task_begin) ++j;
    const AssignJob& jb = b.job[j];
    if (j != cur) {
      __syncthreads();
      const uint4* src = reinterpret_cast<const uint4*>(jb.lut);
      uint4* dst = reinterpret_cast<uint4*>(lut);
#pragma unroll
      for (int i = 0; i < kLutBytes / 16 / kBlock; ++i) dst[tid + i * kBlock] = src[tid + i * kBlock];
      if (tid < 2 * n) tab[tid / n][tid % n] = jb.tables[tid];
      __syncthreads();
      cur = j;
    }
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
      assign_row<WITH_ERR>(jb, lut, tab, n, g8, s8, S, r, c0, active, Ik);
    }
  }
}

hipError_t launch_assign(const AssignBatch& b, bool with_err, hipStream_t stream) {
  const int64_t want = (int64_t)device_cu_count() * 4;
  const int grid = (int)(b.total_tasks < want ? b.total_tasks : want);
  if (grid <= 0) return hipSuccess;
  if (with_err)
    hipLaunchKernelGGL(assign_kernel<true>, dim3(grid), dim3(kBlock), 0, stream, b);
  else
    hipLaunchKernelGGL(assign_kernel<false>, dim3(grid), dim3(kBlock), 0, stream, b);
  return hipGetLastError();
}

}  // namespace aaac
