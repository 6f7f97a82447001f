// Assign step (AAAC summary §2 mechanisms 2 and 4): nearest entries in both tables, selection of
// the table with the lower activation-weighted error, selected codes and selectors written out.
// The lookup structure, the per-weight search and the selection are in lookup.h; the wide
// mapping's row and task walk in assign_body.h.
//
// Work split: workgroup b owns a contiguous range of tasks (rows x one column slab of one matrix);
// each of its waves issues the loads of all its rows of a task before it processes the first one,
// and the workgroup rebuilds the lookup structure in LDS whenever it moves to another matrix. Two
// mappings: 16 weights per lane for selection groups of 16 or more, 8 weights per lane otherwise.
#include "assign_body.h"

namespace aaac {

namespace {

struct RowOut {
  double D;         // E_1 - E_0 of the lane's selection group (after the butterfly)
  double E0, E1;    // E0 with kErrTotal and kErrFull, E1 with kErrFull
  uint32_t P, Q;    // code bytes (q0 | q1 << 4) of weights 0-3 and 4-7
};

// Exact fallback for one lane: full scan of both tables on scaled operands (w and s multiplied by a
// power of two that brings s into [1, 4), so no residual under- or overflows).
template <bool WITH_ERR>
__device__ __forceinline__ void slow_lane(const float* w, uint32_t amax, const float* Ik,
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

// One row of the 8-weight mapping: codes, selection, stores. Returns this lane's share of the
// row's chosen error (its own error sum for the table its group chose; 0 for inactive lanes and
// with kErrNone).
template <int EM, int G8, int S8>
__device__ __forceinline__ double assign_row(const AssignJob& jb, const Lut& lut, int n, int g8,
                                             int s8, int log2S, int64_t base, bool active,
                                             const uint4& v, const float (&Ik)[8]) {
  const uint32_t amax = block_max_u32_t<G8>(lane_absmax_bits(v), g8);
  const float s = __uint_as_float(amax << 16);
  float w[8];
  unpack8(v, w);
  const bool zero = (s == 0.0f);
  const bool fast_scale = zero || (s >= kFastScaleMin && s <= kFastScaleMax);
  const float se = zero ? 1.0f : s;
  const float Y = lut_y(se);
  const float nse = -se;

  float acc = 0.0f, a0 = 0.0f, a1 = 0.0f;
  double accd = 0.0, e0d = 0.0, e1d = 0.0;
  uint32_t Pw = 0, Qw = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    // byte 0 of the lookup's result is the code byte
    const uint32_t c = lookup_weight<EM>(w[k], Y, nse, lut, Ik[k], acc, a0, a1) & 0xFFu;
    if (k < 4) Pw |= c << (8 * k); else Qw |= c << (8 * (k - 4));
    if (k == 3 || k == 7) {
      accd += (double)acc;
      acc = 0.0f;
      if (EM >= kErrTotal) {
        e0d += (double)a0;
        e1d += (double)a1;
        a0 = 0.0f;
        a1 = 0.0f;
      }
    }
  }
  RowOut o;
  o.D = block_sum_f64_t<S8>(accd, s8);
  o.E0 = EM == kErrFull ? block_sum_f64_t<S8>(e0d, s8) : 0.0;
  o.E1 = EM == kErrFull ? block_sum_f64_t<S8>(e1d, s8) : 0.0;
  o.P = Pw;
  o.Q = Qw;
  double L0 = e0d, L1 = e1d;     // the lane's own error sums
  if (zero) {
    o.D = 0.0;
    o.E0 = 0.0;
    o.E1 = 0.0;
    L0 = 0.0;
    L1 = 0.0;
  }
  const bool bad = active && (!fast_scale || !(fabs(o.D) < __builtin_inf()));
  if (__any(bad)) {
    RowOut so;
    slow_lane<(EM >= kErrTotal)>(w, amax, Ik, lut.tab, n, so);
    const double l0 = so.E0, l1 = so.E1;
    so.D = block_sum_f64_t<S8>(so.D, s8);
    if (EM == kErrFull) {
      so.E0 = block_sum_f64_t<S8>(so.E0, s8);
      so.E1 = block_sum_f64_t<S8>(so.E1, s8);
    }
    if (bad) {
      o = so;
      L0 = l0;
      L1 = l1;
    }
  }
  const uint32_t sel = (o.D < 0.0) ? 1u : 0u;
  const uint32_t sh = sel ? 4u : 0u;
  uint32_t p = (o.P >> sh) & 0x0F0F0F0Fu;
  uint32_t q = (o.Q >> sh) & 0x0F0F0F0Fu;
  p |= p >> 4;
  q |= q >> 4;
  const uint32_t packed = __builtin_amdgcn_perm(q, p, 0x06040200u);
  const bool leader = active && ((base >> 3) & (s8 - 1)) == 0;
  if (active) {
    jb.codes[base >> 3] = packed;
    if (leader) {
      const int64_t h = base >> log2S;
      jb.sel[h] = (uint8_t)sel;
      if (EM == kErrFull && jb.err) {
        jb.err[2 * h] = o.E0;
        jb.err[2 * h + 1] = o.E1;
      }
    }
  }
  if (EM == kErrNone || !active) return 0.0;
  return sel ? L1 : L0;
}

}  // namespace

template <int EM, int G16, int S16>
__global__ __launch_bounds__(kBlock, 3) void assign_wide_kernel(AssignBatch b) {
  __shared__ Lut lut;
  __shared__ LutScratch ls;
  assign_wide_body<EM, G16, S16>(b, lut, ls, WholeBlock());
}

template <int EM, int G8, int S8>
__global__ __launch_bounds__(kBlock) void assign_kernel(AssignBatch b) {
  __shared__ Lut lut;
  __shared__ LutScratch ls;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int g8 = b.g / kPerLane, s8 = b.S / kPerLane, n = b.n;
  const int log2S = 31 - __builtin_clz((unsigned)b.S);
  const bool totals = EM == kErrTotal || (EM == kErrFull && b.totals);
  const int64_t t_end = task_lo(blockIdx.x + 1, b.total_tasks, gridDim.x);
  int cur = -1;
  double etot = 0.0;
  for (int64_t task = task_lo(blockIdx.x, b.total_tasks, gridDim.x); task < t_end; ++task) {
    int j = 0;
    while (j + 1 < b.njobs && task >= b.job[j + 1].geom.task_begin) ++j;
    const AssignJob& jb = b.job[j];
    if (j != cur) {
      if (EM != kErrNone && totals && cur >= 0) {
        finish_err_total(b, cur, etot, WholeBlock());
        etot = 0.0;
      }
      __syncthreads();
      build_lut<kBlock>(jb.tables, n, lut, ls);
      cur = j;
    }
    const int64_t local = task - jb.geom.task_begin;
    const int64_t rb = local / jb.geom.nslab;
    const int slab = (int)(local - rb * jb.geom.nslab);
    const int c0 = slab * kSlab + lane * kPerLane;
    const bool active = c0 < jb.geom.C;
    const int64_t R = jb.geom.R, C = jb.geom.C;
    const int64_t r0 = rb * kRowsPerTask + wave;
    // issue the loads of every row of this task first
    uint4 v[kRowsPerWave];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      const int64_t r = r0 + (int64_t)kWavesPerBlock * i;
      v[i] = make_uint4(0u, 0u, 0u, 0u);
      if (active && r < R) v[i] = *reinterpret_cast<const uint4*>(jb.W + r * C + c0);
    }
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
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      const int64_t r = r0 + (int64_t)kWavesPerBlock * i;
      if (r < R) {
        const double e =
            assign_row<EM, G8, S8>(jb, lut, n, g8, s8, log2S, r * C + c0, active, v[i], Ik);
        if (EM != kErrNone) etot += e;
      }
    }
  }
  if (EM != kErrNone && totals && cur >= 0) finish_err_total(b, cur, etot, WholeBlock());
}

// Grid of a launch: enough workgroups to fill every CU at the kernel's occupancy, at most one per
// task and at most kMaxAssignBlocks. With totals, the jobs' workgroup ranges are recorded first.
template <class K>
hipError_t launch_with_grid(K kernel, const AssignBatch& b0, int& occ, hipStream_t stream) {
  if (occ <= 0) {
    int blocks = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, kernel, kBlock, 0);
    occ = (e == hipSuccess && blocks > 0) ? blocks : 2;
  }
  int64_t want = (int64_t)device_cu_count() * occ;
  if (want > kMaxAssignBlocks) want = kMaxAssignBlocks;
  const int grid = (int)(b0.total_tasks < want ? b0.total_tasks : want);
  if (grid <= 0) return hipSuccess;
  AssignBatch b = b0;
  if (b.totals) b.slots = job_slots(b.job, b.njobs, b.total_tasks, grid);
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(kBlock), 0, stream, b);
  return hipGetLastError();
}

template <int EM, int G8, int S8>
hipError_t launch_assign_t(const AssignBatch& b, hipStream_t stream) {
  static int occ = 0;
  return launch_with_grid(assign_kernel<EM, G8, S8>, b, occ, stream);
}

template <int EM, int G16, int S16>
hipError_t launch_assign_wide_t(const AssignBatch& b, hipStream_t stream) {
  static int occ = 0;
  return launch_with_grid(assign_wide_kernel<EM, G16, S16>, b, occ, stream);
}

template <int EM>
hipError_t launch_assign_g(const AssignBatch& b, hipStream_t stream) {
  if (b.S >= kWideLane) {
    // same jobs, task numbering of the wide mapping
    AssignBatch w = b;
    int64_t tb = 0;
    for (int i = 0; i < w.njobs; ++i) {
      w.job[i].geom = make_geom(b.job[i].geom.R, b.job[i].geom.C, tb, kWideSlab,
                                kWideRowsPerTask);
      tb += w.job[i].geom.ntasks;
    }
    w.total_tasks = tb;
    const int g16 = b.g / kWideLane, s16 = b.S / kWideLane;
    if (g16 == 8 && s16 == 8) return launch_assign_wide_t<EM, 8, 8>(w, stream);   // 128/128
    if (g16 == 8 && s16 == 1) return launch_assign_wide_t<EM, 8, 1>(w, stream);   // 128/16
    if (g16 == 1 && s16 == 1) return launch_assign_wide_t<EM, 1, 1>(w, stream);   // 16/16
    return launch_assign_wide_t<EM, 0, 0>(w, stream);
  }
  const int g8 = b.g / kPerLane, s8 = b.S / kPerLane;
  if (g8 == 16 && s8 == 16) return launch_assign_t<EM, 16, 16>(b, stream);
  return launch_assign_t<EM, 0, 0>(b, stream);
}

hipError_t launch_assign(const AssignBatch& b, bool with_err, hipStream_t stream) {
  if (with_err) return launch_assign_g<kErrFull>(b, stream);
  return b.totals ? launch_assign_g<kErrTotal>(b, stream) : launch_assign_g<kErrNone>(b, stream);
}

}  // namespace aaac
