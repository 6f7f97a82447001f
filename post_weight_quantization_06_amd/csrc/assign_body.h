// Device code of the wide assign mapping (16 weights per lane): one row's codes, selections and
// stores, the per-matrix error totals, and a workgroup's walk over its tasks. AAAC summary §2
// mechanisms 2 and 4; the search itself is in lookup.h.
#ifndef AAAC_ASSIGN_BODY_H
#define AAAC_ASSIGN_BODY_H

#include "lookup.h"

namespace aaac {

namespace {

// Sum of this workgroup's chosen errors over job j, then (last workgroup of the job, by an integer
// ticket) the job's total: each lane's running sum in row order, the lanes of a wave by butterfly,
// the waves in order, the workgroups' partials in workgroup order. Every order is fixed, so the
// total is reproducible for a given call. Called by every thread of the group pt (barriers).
template <class Part>
__device__ void finish_err_total(const AssignBatch& b, int j, double lane_sum, Part pt) {
  __shared__ double wsum[kWavesPerBlock];
  __shared__ uint32_t ticket;
  const int tid = pt.tid(), lane = tid & (kWave - 1), wave = tid / kWave;
  const AssignJob& jb = b.job[j];
  double* part = b.partials + (size_t)j * b.slots;
  const double ws = block_sum_f64_t<kWave>(lane_sum, kWave);
  pt.sync();
  if (lane == 0) wsum[wave] = ws;
  pt.sync();
  if (tid == 0) {
    part[(int)blockIdx.x - jb.wg_lo] = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
    __threadfence();
    ticket = atomicAdd(b.counters + j, 1u);
  }
  pt.sync();
  if (ticket != (uint32_t)(jb.wg_count - 1)) return;
  // last workgroup of this job: every partial is visible after the fence
  __threadfence();
  const int cnt = jb.wg_count;
  const int s0 = (tid * cnt) / kBlock, s1 = ((tid + 1) * cnt) / kBlock;
  double acc = 0.0;
  for (int i = s0; i < s1; ++i) acc += part[i];
  const double t = block_sum_f64_t<kWave>(acc, kWave);
  pt.sync();
  if (lane == 0) wsum[wave] = t;
  pt.sync();
  if (tid == 0) {
    *jb.err_total = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
    b.counters[j] = 0u;
  }
}

template <int EM, int G16, int S16>
__device__ __forceinline__ double assign_row16(const AssignJob& jb, const Lut& lut, int n,
                                               int g16, int s16, int log2S, int64_t r, int c0,
                                               bool active, const uint16_t* wsafe,
                                               const float* isafe, const uint4& va,
                                               const uint4& vb, const float (&Ik)[16]) {
  Row16 o;
  row16_core<EM, G16, S16>(lut, n, g16, s16, active, wsafe, isafe, va, vb, Ik, o);
  const int64_t rc = r * jb.geom.C;          // wave-uniform; a multiple of S
  if (active)
    store_row16<EM>(o, jb.codes + (rc >> 3), jb.sel + (rc >> log2S),
                    (EM == kErrFull && jb.err) ? jb.err + 2 * (rc >> log2S) : nullptr, s16, log2S,
                    c0);
  return (EM != kErrNone && active) ? o.Esel : 0.0;
}

// The wide kernel's work for one workgroup, with the lookup structure in lut; pt names the kBlock
// threads that run it.
template <int EM, int G16, int S16, class Part>
__device__ __forceinline__ void assign_wide_body(const AssignBatch& b, Lut& lut, LutScratch& ls,
                                                 Part pt) {
  const int lane = pt.tid() & (kWave - 1);
  const int wave = pt.wave();
  const int g16 = b.g / kWideLane, s16 = b.S / kWideLane, n = b.n;
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
        finish_err_total(b, cur, etot, pt);
        etot = 0.0;
      }
      pt.sync();
      build_lut<kBlock>(jb.tables, n, lut, ls, pt);
      cur = j;
    }
    const int64_t local = task - jb.geom.task_begin;
    const int64_t rb = local / jb.geom.nslab;
    const int slab = (int)(local - rb * jb.geom.nslab);
    const int c0 = slab * kWideSlab + lane * kWideLane;
    const bool active = c0 < jb.geom.C;
    const int cl = active ? c0 : 0;           // inactive lanes read an element of their own matrix
    const int64_t R = jb.geom.R, C = jb.geom.C;
    const int64_t r0 = rb * kWideRowsPerTask + wave;
    // every load of the task first, unconditional (rows past the end read the last row and are
    // skipped below; that test is the same for the whole wave)
    uint4 va[kWideRowsPerWave], vb[kWideRowsPerWave];
#pragma unroll
    for (int i = 0; i < kWideRowsPerWave; ++i) {
      int64_t r = r0 + (int64_t)kWavesPerBlock * i;
      r = r < R ? r : R - 1;
      const uint16_t* p = jb.W + r * C;         // wave-uniform row base
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
      const double e = assign_row16<EM, G16, S16>(jb, lut, n, g16, s16, log2S, r, c0, active,
                                                  jb.W + r * C + cl, jb.I + cl, va[i], vb[i], Ik);
      if (EM != kErrNone) etot += e;
    }
  }
  if (EM != kErrNone && totals && cur >= 0) finish_err_total(b, cur, etot, pt);
}

}  // namespace
}  // namespace aaac

#endif  // AAAC_ASSIGN_BODY_H
