// Lookup structure and per-row nearest-entry search shared by the assign kernel and the fused
// assign + accumulate kernel (AAAC summary §2 mechanisms 2 and 4).
//
// For every weight w of a scale group with scale s = max|w| and each table c, the nearest entry
// q_c minimizes |u - T_c[j]| with u = w / s, ties to the lower index. Because s > 0 this is the
// same as minimizing |w - s T_c[j]|, and it is decided on r = fma(-s, T, w), the exactly rounded
// residual: when the rounded magnitudes differ, the exact ones differ the same way, and when they
// are equal the two squared distances agree to 2^-22 relative. Candidates come from a 1024-record
// table indexed by an approximate u, built so that each record lists every entry that can be
// nearest anywhere in (a slightly widened copy of) its interval; a record that would need more than
// two candidates routes its group to an exact full scan.
//
// Per selection group, D = E_1 - E_0 = sum I_k (m_1^2 - m_0^2) with m_c the chosen residual
// magnitude: fp32 over four weights, then fp64. The selection is D < 0 (ties keep T0). Its
// rounding error is below 8 * 2^-24 (E_0 + E_1), so a selection can only differ from the exact one
// when |E_1 - E_0| < 1e-6 max(E_0, E_1).
//
// Error outputs (template parameter EM): kErrNone computes only D. kErrTotal also sums I m_0^2 and
// I m_1^2 over each lane's weights (fp32 over four weights, then fp64; no reduction across lanes):
// once the group's selection is known, each lane's share of the chosen error is its own sum for
// the chosen table, so a matrix's total is the sum of every lane's share (no cancellation). kErrFull
// also reduces E_0 and E_1 over each group for the error array.
#ifndef AAAC_LOOKUP_H
#define AAAC_LOOKUP_H

#include "common.h"

namespace aaac {

constexpr int kErrNone = 0;
constexpr int kErrTotal = 1;
constexpr int kErrFull = 2;

namespace {

struct LutScratch {
  float raw[2][16];
  int first[2][16];
  float sv[2][16];          // distinct values, ascending
  int six[2][16];           // lowest index holding each distinct value
  int m[2];                 // distinct values (0: the table has a non-finite entry)
  uint32_t wsum[16];        // per-wave totals of the record scan
};

// The lookup structure in LDS: per record one word, (i0 | i1 << 4) | off << 8: the code base and
// the byte offset of the record's candidates in `combo`, whose entry (p0, p1) holds pair p0 of
// table 0 and pair p1 of table 1, {T0[p0], T0[p0 + 1], T1[p1], T1[p1 + 1]} (one 16-byte read per
// weight gives all four candidates). The per-table pair arrays are kept for building it.
struct Lut {
  uint32_t rec[kLutRecs];
  float4 combo[kPairs * kPairs];
  float2 pairs[2][kPairs];
  float tab[2][16];         // the raw tables, for the exact scan
};

// Build the lookup structure for tables T (fp32 [2][n], global) with the NT threads of the group pt
// (a power of two from 64 to 1024). Must be called by every thread of the group; ends with the
// group's barrier.
//
// Midpoint i of a table (between its distinct values i and i + 1) lies in the records
// [mlo_i, mhi_i] and below every record past mhi_i. Per record, "below" (midpoints below it) and
// "inside" (midpoints in it) decide the candidates. They are counted with a difference array: each
// midpoint adds +1 to below at mhi_i + 1, +1 to inside at mlo_i and -1 at mhi_i + 1, one byte per
// count in a packed word (below_0, inside_0, below_1, inside_1; every count is at most 15, so the
// packed prefix sums are exact). The array lives in the record words themselves, and one prefix
// scan over the 1024 records turns it into the counts, which each thread then replaces by its
// records' final words.
template <int NT, class Part = WholeBlock>
__device__ __noinline__ void build_lut(const float* __restrict__ T, int n, Lut& lut, LutScratch& ls,
                                       Part pt = Part()) {
  static_assert(NT >= kWave && NT <= kLutRecs && (NT & (NT - 1)) == 0, "block size");
  const int tid = pt.tid();
  const float qnan = __uint_as_float(0x7fc00000u);
  if (tid < 32) {
    const int c = tid >> 4, j = tid & 15;
    const float x = j < n ? T[c * n + j] : 0.0f;
    ls.raw[c][j] = x;
    lut.tab[c][j] = x;
  }
  constexpr int kPer = kLutRecs / NT;       // records per thread
#pragma unroll
  for (int k = 0; k < kPer; ++k) lut.rec[tid + NT * k] = 0u;
  pt.sync();
  if (tid < 32) {
    const int c = tid >> 4, j = tid & 15;
    const float x = ls.raw[c][j];
    bool first = j < n;
    for (int k = 0; k < j; ++k) first = first && !(ls.raw[c][k] == x);
    ls.first[c][j] = first ? 1 : 0;
    // pair j: {T[j], T[j + 1]}, the entry past the end reads as +inf
    const float nxt = (j + 1 < n) ? ls.raw[c][j + 1 < 16 ? j + 1 : 15] : __builtin_inff();
    lut.pairs[c][j] = make_float2(j < n ? x : __builtin_inff(), nxt);
    if (j < 2) lut.pairs[c][16 + j] = j == 0 ? make_float2(__builtin_inff(), __builtin_inff())
                                             : make_float2(qnan, qnan);
  }
  pt.sync();
  // every combination of a table-0 pair and a table-1 pair
  for (int e = tid; e < kPairs * kPairs; e += NT) {
    const float2 a = lut.pairs[0][e / kPairs], b = lut.pairs[1][e % kPairs];
    lut.combo[e] = make_float4(a.x, a.y, b.x, b.y);
  }
  if (tid < 32) {
    const int c = tid >> 4, j = tid & 15;
    const float x = ls.raw[c][j];
    int rank = 0, m = 0;
    bool finite = true;
    for (int k = 0; k < n; ++k) {
      const float y = ls.raw[c][k];
      finite = finite && isfinite(y);
      if (ls.first[c][k]) {
        ++m;
        if (y < x) ++rank;
      }
    }
    if (ls.first[c][j] && finite) {
      ls.sv[c][rank] = x;
      ls.six[c][rank] = j;
    }
    if (j == 0) ls.m[c] = finite ? m : 0;
  }
  pt.sync();
  if (tid < 32) {
    const int c = tid >> 4, i = tid & 15;
    if (i + 1 < ls.m[c]) {
      const double M = 0.5 * ((double)ls.sv[c][i] + (double)ls.sv[c][i + 1]);
      const double S = (double)kLutScale;
      const double hi = floor((M + 1.0 + kLutSlack) * S + 1.5);
      const double lo = ceil((M + 1.0 - kLutSlack) * S + 0.5);
      // hi >= lo always; both clamped to [-1, 4096]
      const int mhi = (int)fmin(fmax(hi, -1.0), 4096.0);
      const int mlo = (int)fmin(fmax(lo, -1.0), 4096.0);
      const int end = mhi + 1;                           // >= 0
      const bool in_range = mhi >= 0 && mlo < kLutRecs;  // the midpoint lies in some record
      const uint32_t in1 = 1u << (16 * c + 8);
      if (end < kLutRecs) atomicAdd(&lut.rec[end], (1u << (16 * c)) - (in_range ? in1 : 0u));
      if (in_range) atomicAdd(&lut.rec[mlo > 0 ? mlo : 0], in1);
    }
  }
  pt.sync();
  // prefix sums: thread t owns the run of kPer consecutive records starting at t * kPer
  const int r0 = tid * kPer;
  uint32_t tot = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) tot += lut.rec[r0 + k];
  // inclusive scan of the thread totals within the wave, then across the waves
  const int lane = tid & (kWave - 1);
  uint32_t incl = tot;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const uint32_t o = (uint32_t)__shfl_up((int)incl, d);
    if (lane >= d) incl += o;
  }
  if (lane == kWave - 1) ls.wsum[tid / kWave] = incl;
  pt.sync();
  uint32_t P = incl - tot;
  const int wv = tid / kWave;
#pragma unroll
  for (int w = 0; w < NT / kWave - 1; ++w) P += (w < wv) ? ls.wsum[w] : 0u;
  // each record is read (its difference) before this thread overwrites it with the final word
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    P += lut.rec[r0 + k];
    uint32_t pi[2];
    uint32_t code = 0;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int m = ls.m[c];
      const int below = (int)((P >> (16 * c)) & 0xFFu);
      const int inside = (int)((P >> (16 * c + 8)) & 0xFFu);
      // clamped indices keep every read inside the arrays whatever the branch
      const int j0 = below < 15 ? below : 15;
      const int j1 = below + 1 < 15 ? below + 1 : 15;
      // one candidate: pair {T[i], T[i + 1]} whose second entry is never strictly nearer inside
      // the record; two candidates: only when they are consecutive entries i, i + 1
      const bool single = m > 0 && inside == 0;
      const bool pair = m > 0 && inside == 1 && ls.six[c][j1] == ls.six[c][j0] + 1;
      const int i0 = ls.six[c][j0];
      pi[c] = (uint32_t)((single || pair) ? i0 : kNaNPair);
      code |= (single || pair) ? ((uint32_t)i0 << (4 * c)) : 0u;
    }
    lut.rec[r0 + k] = code | (((pi[0] * kPairs + pi[1]) * (uint32_t)sizeof(float4)) << 8);
  }
  pt.sync();
}

// Y for a group scale se > 0 (the lookup's u = w / se, scaled into the record index).
__device__ __forceinline__ float lut_y(float se) { return kLutY * __builtin_amdgcn_rcpf(se); }

// The lookup of one weight in two steps, so that callers can issue every record read of a row
// before the candidate reads: the record word of w, then (from that word) the four candidates.
__device__ __forceinline__ uint32_t lut_record(float w, float Y, const Lut& lut) {
  const float t = __builtin_fmaf(w, Y, kLutMagic);
  const uint32_t ra = __float_as_uint(t) << 2;
  return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(lut.rec) + ra);
}

__device__ __forceinline__ float4 lut_candidates(uint32_t rec, const Lut& lut) {
  return *reinterpret_cast<const float4*>(reinterpret_cast<const uint8_t*>(lut.combo) +
                                          (rec >> 8));
}

// Nearest entries of one weight in both tables from its record word and candidates: returns the
// record word with the code byte q0 | q1 << 4 in byte 0 (the increments never carry out of a
// nibble: a pair whose second entry is past the table or NaN is never taken), and accumulates
// I (m1^2 - m0^2) (and I m0^2, I m1^2 as EM asks).
template <int EM>
__device__ __forceinline__ uint32_t lut_decide(float w, float nse, uint32_t rec, const float4& p,
                                               float Ik, float& acc, float& a0, float& a1) {
  const float r0a = __builtin_fmaf(nse, p.x, w);
  const float r0b = __builtin_fmaf(nse, p.y, w);
  const float r1a = __builtin_fmaf(nse, p.z, w);
  const float r1b = __builtin_fmaf(nse, p.w, w);
  const bool d0 = fabsf(r0b) < fabsf(r0a);
  const bool d1 = fabsf(r1b) < fabsf(r1a);
  const float m0 = fminf(fabsf(r0a), fabsf(r0b));
  const float m1 = fminf(fabsf(r1a), fabsf(r1b));
  const float e0 = m0 * m0;
  acc = __builtin_fmaf(Ik, __builtin_fmaf(m1, m1, -e0), acc);
  if (EM >= kErrTotal) {
    a0 = __builtin_fmaf(Ik, e0, a0);
    a1 = __builtin_fmaf(Ik, m1 * m1, a1);
  }
  return rec + (d0 ? 1u : 0u) + (d1 ? 16u : 0u);   // byte 0: the code byte
}

// Both steps for one weight (see the layout above).
template <int EM>
__device__ __forceinline__ uint32_t lookup_weight(float w, float Y, float nse, const Lut& lut,
                                                  float Ik, float& acc, float& a0, float& a1) {
  const uint32_t rec = lut_record(w, Y, lut);
  return lut_decide<EM>(w, nse, rec, lut_candidates(rec, lut), Ik, acc, a0, a1);
}

// Exact fallback for one lane of the wide mapping, reading its 16 weights and importances again
// from memory (they are in cache) so that the fast path keeps no copies in registers: full scan of
// both tables on operands scaled by a power of two that brings s into [1, 4). Codes come back as
// bytes q0 | q1 << 4, weight k in byte k of (lo, hi).
template <bool WITH_ERR>
__device__ __noinline__ void slow_lane16(const uint16_t* __restrict__ wp,
                                         const float* __restrict__ ip, uint32_t amax,
                                         const float (*tab)[16], int n, double& D, double& E0,
                                         double& E1, uint64_t& lo, uint64_t& hi) {
  const uint32_t E = min(max(amax >> 7, 1u), 253u);
  const float P = __uint_as_float((254u - E) << 23);
  const float sp = __uint_as_float(amax << 16) * P;
  double d = 0.0, e0 = 0.0, e1 = 0.0;
  uint64_t cl = 0, ch = 0;
#pragma unroll 1
  for (int k = 0; k < kWideLane; ++k) {
    const float wv = __uint_as_float((uint32_t)wp[k] << 16) * P;
    const double Ik = (double)ip[k];
    float best0 = __builtin_inff(), best1 = __builtin_inff();
    uint32_t q0 = 0, q1 = 0;
    for (int j = 0; j < n; ++j) {
      const float r0 = fabsf(__builtin_fmaf(-sp, tab[0][j], wv));
      const float r1 = fabsf(__builtin_fmaf(-sp, tab[1][j], wv));
      if (r0 < best0) { best0 = r0; q0 = j; }
      if (r1 < best1) { best1 = r1; q1 = j; }
    }
    const double b0 = (double)best0 * (double)best0;
    const double b1 = (double)best1 * (double)best1;
    d += Ik * (b1 - b0);
    if (WITH_ERR) {
      e0 += Ik * b0;
      e1 += Ik * b1;
    }
    const uint64_t c = (uint64_t)(q0 | (q1 << 4));
    if (k < 8) cl |= c << (8 * k); else ch |= c << (8 * (k - 8));
  }
  const double inv = 1.0 / ((double)P * (double)P);
  D = d;
  E0 = e0 * inv;
  E1 = e1 * inv;
  lo = cl;
  hi = ch;
}

// Codes, selection and errors of one row of the wide mapping (16 weights per lane); nothing is
// stored. The code bytes q0 | q1 << 4 are gathered by column parity so that the chosen nibbles
// pack into code words with one bit-field insert: E[h] byte b belongs to weight 8h + 2b, O[h]
// byte b to weight 8h + 2b + 1.
struct Row16 {
  uint32_t E[2], O[2];
  uint32_t sel;      // 1 = T1
  float s;           // the group scale (0 for an all-zero group)
  double E0, E1;     // group errors (kErrFull)
  double Esel;       // this lane's share of the row's chosen error (kErrTotal, kErrFull)
};

// The scale of one row of the wide mapping: the lane's 16 weights unpacked, the group's largest
// |w| (as an fp32 bit pattern: a bf16 value, low 16 bits zero), and the lookup constants.
struct Row16Scale {
  float s, Y, nse;
  uint32_t amax;       // s as bf16 bits
  bool zero;           // all-zero group
  bool fast_scale;     // s within the range where the lookup's residuals are exact
};

template <int G16>
__device__ __forceinline__ void row16_scale(const uint4& va, const uint4& vb, int g16,
                                            float (&w)[16], Row16Scale& sc) {
  {
    float wa[8], wb[8];
    unpack8(va, wa);
    unpack8(vb, wb);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      w[k] = wa[k];
      w[8 + k] = wb[k];
    }
  }
  const uint32_t sbits = block_max_u32_t<G16>(absmax16_f32_bits(w), g16);
  sc.amax = sbits >> 16;
  sc.s = __uint_as_float(sbits);
  sc.zero = (sc.s == 0.0f);
  // bitwise, not short-circuit: a branch here would split the row's schedule in two
  sc.fast_scale = sc.zero | ((sc.s >= kFastScaleMin) & (sc.s <= kFastScaleMax));
  const float se = sc.zero ? 1.0f : sc.s;
  sc.Y = lut_y(se);
  sc.nse = -se;
}

// The rest of a row once every weight's code word c[k] (code byte in byte 0) and the lane's
// partial sums are known: gather the codes, reduce D over the selection group, take the exact
// scan where needed, select. wsafe / isafe address the lane's 16 weights and importances in memory
// (in bounds also for inactive lanes) for the exact fallback.
template <int EM, int S16>
__device__ __forceinline__ void row16_finish(const Lut& lut, int n, int s16, bool active,
                                             const uint16_t* wsafe, const float* isafe,
                                             const uint32_t (&c)[16], double accd, double e0d,
                                             double e1d, const Row16Scale& sc, Row16& o) {
  // byte 0 of c[k] is weight k's code byte; gather them by column parity
  uint32_t Ew[2], Ow[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t* ch = c + 8 * h;
    const uint32_t e01 = __builtin_amdgcn_perm(ch[2], ch[0], 0x0c0c0400u);
    const uint32_t e23 = __builtin_amdgcn_perm(ch[6], ch[4], 0x0c0c0400u);
    Ew[h] = __builtin_amdgcn_perm(e23, e01, 0x05040100u);
    const uint32_t o01 = __builtin_amdgcn_perm(ch[3], ch[1], 0x0c0c0400u);
    const uint32_t o23 = __builtin_amdgcn_perm(ch[7], ch[5], 0x0c0c0400u);
    Ow[h] = __builtin_amdgcn_perm(o23, o01, 0x05040100u);
  }
  double D = block_sum_f64_t<S16>(accd, s16);
  // the lane's own error sums (kErrTotal, kErrFull); kErrFull also reduces them over the group
  double L0 = e0d, L1 = e1d;
  double E0 = EM == kErrFull ? block_sum_f64_t<S16>(e0d, s16) : 0.0;
  double E1 = EM == kErrFull ? block_sum_f64_t<S16>(e1d, s16) : 0.0;
  if (sc.zero) {
    D = 0.0;
    E0 = 0.0;
    E1 = 0.0;
    L0 = 0.0;
    L1 = 0.0;
  }
  const bool bad = active && (!sc.fast_scale || !(fabs(D) < __builtin_inf()));
  if (__any(bad)) {
    double lD, lE0, lE1;
    uint64_t clo, chi;
    slow_lane16<(EM >= kErrTotal)>(wsafe, isafe, sc.amax, lut.tab, n, lD, lE0, lE1, clo, chi);
    const double sD = block_sum_f64_t<S16>(lD, s16);
    double sE0 = 0.0, sE1 = 0.0;
    if (EM == kErrFull) {
      sE0 = block_sum_f64_t<S16>(lE0, s16);
      sE1 = block_sum_f64_t<S16>(lE1, s16);
    }
    if (bad) {
      D = sD;
      E0 = sE0;
      E1 = sE1;
      L0 = lE0;
      L1 = lE1;
      // byte k of (clo, chi) is weight k
      const uint32_t l0 = (uint32_t)clo, l1 = (uint32_t)(clo >> 32);
      const uint32_t h0 = (uint32_t)chi, h1 = (uint32_t)(chi >> 32);
      Ew[0] = __builtin_amdgcn_perm(l1, l0, 0x06040200u);
      Ow[0] = __builtin_amdgcn_perm(l1, l0, 0x07050301u);
      Ew[1] = __builtin_amdgcn_perm(h1, h0, 0x06040200u);
      Ow[1] = __builtin_amdgcn_perm(h1, h0, 0x07050301u);
    }
  }
  o.E[0] = Ew[0]; o.E[1] = Ew[1];
  o.O[0] = Ow[0]; o.O[1] = Ow[1];
  o.sel = (D < 0.0) ? 1u : 0u;
  o.s = sc.s;
  o.E0 = E0;
  o.E1 = E1;
  o.Esel = o.sel ? L1 : L0;
}

// One row: group scale, nearest entries of all sixteen weights, and the selection of each group.
// G16 / S16 are the lanes per scale / selection group (0: the runtime g16 / s16). The compiler
// may interleave all sixteen lookups (the exact scan is out of line, so the row stays within the
// register budget of four waves per SIMD).
template <int EM, int G16, int S16>
__device__ __forceinline__ void row16_core(const Lut& lut, int n, int g16, int s16, bool active,
                                           const uint16_t* wsafe, const float* isafe,
                                           const uint4& va, const uint4& vb,
                                           const float (&Ik)[16], Row16& o) {
  float w[16];
  Row16Scale sc;
  row16_scale<G16>(va, vb, g16, w, sc);
  uint32_t c[16];
  double accd = 0.0, e0d = 0.0, e1d = 0.0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    // four weights per fp32 partial, then fp64
    float acc = 0.0f, a0 = 0.0f, a1 = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      c[4 * q + k] =
          lookup_weight<EM>(w[4 * q + k], sc.Y, sc.nse, lut, Ik[4 * q + k], acc, a0, a1);
    accd = (q == 0) ? (double)acc : accd + (double)acc;
    if (EM >= kErrTotal) {
      e0d = (q == 0) ? (double)a0 : e0d + (double)a0;
      e1d = (q == 0) ? (double)a1 : e1d + (double)a1;
    }
  }
  row16_finish<EM, S16>(lut, n, s16, active, wsafe, isafe, c, accd, e0d, e1d, sc, o);
}

// The selected codes of a row as two code words: nibble m of word h is weight 8h + m.
__device__ __forceinline__ uint2 chosen_codes16(const Row16& o) {
  const uint32_t sh = o.sel ? 4u : 0u;
  uint32_t out[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    // low nibble: the chosen code of the even column, high nibble: of the odd column
    const uint32_t lo = o.E[k] >> sh;
    const uint32_t hi = o.O[k] << (4u - sh);
    out[k] = (lo & 0x0F0F0F0Fu) | (hi & 0xF0F0F0F0u);
  }
  return make_uint2(out[0], out[1]);
}

// Store the selected codes (8 bytes), and once per selection group the selector (and errors).
// codes_row, sel_row and err_row point at the row's first code word, selector and error pair
// (wave-uniform); c0 is the lane's first column. Rows start on a selection-group boundary, so the
// lane's offsets within the row follow from c0 alone.
template <int EM>
__device__ __forceinline__ void store_row16(const Row16& o, uint32_t* codes_row, uint8_t* sel_row,
                                            double* err_row, int s16, int log2S, int c0) {
  *reinterpret_cast<uint2*>(codes_row + (c0 >> 3)) = chosen_codes16(o);
  if (((c0 >> 4) & (s16 - 1)) == 0) {
    const int h = c0 >> log2S;
    sel_row[h] = (uint8_t)o.sel;
    if (EM == kErrFull && err_row) {
      err_row[2 * h] = o.E0;
      err_row[2 * h + 1] = o.E1;
    }
  }
}

}  // namespace
}  // namespace aaac

#endif  // AAAC_LOOKUP_H
