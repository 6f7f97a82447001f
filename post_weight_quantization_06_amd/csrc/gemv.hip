// Decode GEMV on the packed format (AAAC summary §1: 4-bit weights with 16-bit activations, W4A16,
// where the dequantized values are the weights inference uses; §2 mechanism 3: the stored format).
//
//   y[b, r] = sum_c |s(r, c)| T~_sigma(r, c)[q(r, c)] x[b, c]
//
// with the scale factored out of each scale group: y = sum_groups |s| (sum_k T~[q_k] x_k). The
// weight is the exact product of the stored bf16 scale and bf16 entry; the bf16 rounding that
// dequant applies when it stores W_hat never happens here.
//
// Lookup: for every matrix and table the workgroup holds a 256-entry pair table in LDS, indexed by
// a whole code byte: entry b = (T~[b & 15], T~[b >> 4]) as two bf16 (low half = even column), so
// one LDS read serves two weights and feeds one v_dot2 against the matching pair of x values.
//
// Mapping: a lane owns 32 consecutive columns (16 code bytes, one 16-byte load), a wave row covers
// 2048 columns. A wave walks two blocks of 4 rows of one matrix over its share of the slabs, the
// next (block, slab) unit loading while the current one is used, with the x slab in registers and
// one fp32 accumulator per row and batch row. The 64 lane partials of a row are added by a fixed
// butterfly, the wave partials of a split row in wave order, so results are bitwise reproducible.
#include "common.h"

namespace aaac {

namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kGemvLane = 32;                       // columns per lane per slab
constexpr int kGemvSlab = kWave * kGemvLane;        // 2048 columns
constexpr int kGemvRows = 4;                        // rows per row block
constexpr int kPairEntries = 256;

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Loads of one 2048-column slab of a task: codes, scale words and selector bits of every row, and
// the x pairs of the lane's 32 columns. A lane past the last column reads column 0 instead and is
// skipped when the slab is used.
template <int NB, int GPL>
struct Slab {
  uint4 cw[kGemvRows];
  uint32_t sw[kGemvRows][GPL];
  uint32_t sb[kGemvRows];
  uint32_t xw[NB][16];
  bool active;
};

template <int NB, int GPL, int SPL, bool SIGN>
__device__ __forceinline__ void load_slab(const GemvJob& jb, int64_t r0, int64_t cs, int log2g,
                                          int log2S, Slab<NB, GPL>& t) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t R = jb.R, C = jb.C;
  const int64_t c0 = cs + lane * kGemvLane;
  t.active = c0 < C;
  const int cl = t.active ? (int)c0 : 0;
#pragma unroll
  for (int q = 0; q < NB; ++q) {
    const uint4* xp = reinterpret_cast<const uint4*>(jb.x + q * C + cl);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint4 u = xp[v];
      t.xw[q][4 * v] = u.x; t.xw[q][4 * v + 1] = u.y; t.xw[q][4 * v + 2] = u.z;
      t.xw[q][4 * v + 3] = u.w;
    }
  }
#pragma unroll
  for (int i = 0; i < kGemvRows; ++i) {
    const int64_t r = (r0 + i < R) ? r0 + i : R - 1;
    const int64_t rc = r * C;                       // wave-uniform; a multiple of 32
    t.cw[i] = *reinterpret_cast<const uint4*>(jb.codes + (rc >> 1) + (cl >> 1));
    const uint16_t* sp = jb.scales + (rc >> log2g) + (cl >> log2g);
    if (GPL == 1) {
      t.sw[i][0] = sp[0];
    } else if (GPL == 2) {
      const uint32_t v = *reinterpret_cast<const uint32_t*>(sp);
      t.sw[i][0] = v & 0xffffu; t.sw[i][1] = v >> 16;
    } else {
      const uint2 v = *reinterpret_cast<const uint2*>(sp);
      t.sw[i][0] = v.x & 0xffffu; t.sw[i][1] = v.x >> 16;
      t.sw[i][2] = v.y & 0xffffu; t.sw[i][3] = v.y >> 16;
    }
    if (SIGN) {
      uint32_t bits = 0;
#pragma unroll
      for (int k = 0; k < GPL; ++k) bits |= (t.sw[i][k] >> 15) << k;
      t.sb[i] = bits;
    } else {
      const int64_t h = (rc >> log2S) + (cl >> log2S);   // first selection group of the lane row
      t.sb[i] = ((uint32_t)jb.bitmap[h >> 3] >> (h & 7)) & ((1u << SPL) - 1u);
    }
  }
}

// Pair-table entries of one lane row: all 16 reads are issued before any is used, so their LDS
// latencies overlap.
template <int SPL>
__device__ __forceinline__ void fetch_row(const uint4& cw, uint32_t sb, const uint32_t* pj,
                                          uint32_t (&e)[16]) {
  const uint32_t words[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const uint32_t byte = (words[k >> 2] >> (8 * (k & 3))) & 0xffu;
    const uint32_t sig = (sb >> (k / (16 / SPL))) & 1u;
    e[k] = pj[(sig << 8) | byte];
  }
}

template <int NB, int GPL>
__device__ __forceinline__ void dot_row(const uint32_t (&e)[16], const uint32_t (&sw)[GPL],
                                        const uint32_t (&xw)[NB][16], float (&acc)[NB]) {
  float part[NB];
#pragma unroll
  for (int q = 0; q < NB; ++q) part[q] = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
#pragma unroll
    for (int q = 0; q < NB; ++q) part[q] = dot2(e[k], xw[q][k], part[q]);
    if ((k + 1) % (16 / GPL) == 0) {
      const float s = __uint_as_float((sw[k / (16 / GPL)] & 0x7fffu) << 16);
#pragma unroll
      for (int q = 0; q < NB; ++q) {
        acc[q] = fmaf(s, part[q], acc[q]);
        part[q] = 0.0f;
      }
    }
  }
}

// Rows in pairs of buffers: the reads of row i + 1 are in flight while row i is added up.
template <int NB, int GPL, int SPL>
__device__ __forceinline__ void use_slab(const Slab<NB, GPL>& t, const uint32_t* pj,
                                         float (&acc)[kGemvRows][NB]) {
  if (!t.active) return;
  uint32_t ea[16], eb[16];
  fetch_row<SPL>(t.cw[0], t.sb[0], pj, ea);
#pragma unroll
  for (int i = 0; i < kGemvRows; i += 2) {
    fetch_row<SPL>(t.cw[i + 1], t.sb[i + 1], pj, eb);
    dot_row<NB, GPL>(ea, t.sw[i], t.xw, acc[i]);
    if (i + 2 < kGemvRows) fetch_row<SPL>(t.cw[i + 2], t.sb[i + 2], pj, ea);
    dot_row<NB, GPL>(eb, t.sw[i + 1], t.xw, acc[i + 1]);
  }
}

// GPL: scale groups per lane row (g >= 32: 1, g = 16: 2, g = 8: 4); SPL: selection groups per lane
// row, likewise from S; SIGN: the selector is the scale's sign bit (S == g), else the bitmap.
//
// One workgroup task per workgroup (the grid is not persistent, so the dispatcher balances the
// tasks). A task covers two rounds of row blocks of kGemvRows rows: the four waves take one row
// block each per round when the matrix has at most two slabs, else 4 / k row blocks with k waves
// splitting the slabs of each, and the k partial sums of a row are added in wave order through
// LDS. Each wave uses its units (block, slab) in order, loading the next while it uses one.
template <int NB, int GPL, int SPL, bool SIGN>
__global__ __launch_bounds__(kBlock) void gemv_kernel(GemvBatch b) {
  __shared__ uint32_t pairs[2][kPairEntries];
  __shared__ float red[2][kWavesPerBlock][kGemvRows][NB];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = wave_index();
  const int64_t task = blockIdx.x;
  int j = 0;
  while (j + 1 < b.njobs && task >= b.job[j + 1].task_begin) ++j;
  const GemvJob& jb = b.job[j];
  for (int i = tid; i < 2 * kPairEntries; i += kBlock) {
    const int c = i / kPairEntries, e = i & (kPairEntries - 1);
    const uint16_t* t = jb.tables + c * b.n;
    const int lo = e & 15, hi = e >> 4;
    const uint32_t vlo = t[lo < b.n ? lo : 0], vhi = t[hi < b.n ? hi : 0];
    pairs[c][e] = vlo | (vhi << 16);
  }
  __syncthreads();
  const int log2g = 31 - __builtin_clz((unsigned)b.g);
  const int log2S = 31 - __builtin_clz((unsigned)b.S);
  const int64_t R = jb.R, C = jb.C;
  const int k = jb.split;                              // waves per row block: 1, 2 or 4
  const int nslab = (int)((C + kGemvSlab - 1) / kGemvSlab);
  const int per = (nslab + k - 1) / k;
  const int part = wave % k;
  const int groups = kWavesPerBlock / k;
  const int64_t base = (task - jb.task_begin) * 2 * groups * kGemvRows;
  const int64_t r0a = base + (int64_t)(wave / k) * kGemvRows;
  const int64_t r0b = r0a + (int64_t)groups * kGemvRows;
  const int64_t s_begin = (int64_t)part * per * kGemvSlab;
  int64_t s_end = (int64_t)(part + 1) * per * kGemvSlab;
  s_end = s_end < C ? s_end : C;
  const int ns = s_begin < s_end ? (int)((s_end - s_begin + kGemvSlab - 1) / kGemvSlab) : 0;
  const int nu = r0a >= R ? 0 : (r0b >= R ? ns : 2 * ns);
  const uint32_t* pj = &pairs[0][0];
  float acc0[kGemvRows][NB], accT[kGemvRows][NB];
#pragma unroll
  for (int i = 0; i < kGemvRows; ++i)
#pragma unroll
    for (int q = 0; q < NB; ++q) { acc0[i][q] = 0.0f; accT[i][q] = 0.0f; }
  if (nu > 0) {
    Slab<NB, GPL> A, B;
    // unit u: row block u / ns (first or second round), slab u % ns of the share
    auto unit_r = [&](int u) { return u < ns ? r0a : r0b; };
    auto unit_c = [&](int u) { return s_begin + (int64_t)(u % ns) * kGemvSlab; };
    load_slab<NB, GPL, SPL, SIGN>(jb, r0a, s_begin, log2g, log2S, A);
    for (int u = 0; u < nu; u += 2) {
      const int u1 = u + 1 < nu ? u + 1 : nu - 1;
      load_slab<NB, GPL, SPL, SIGN>(jb, unit_r(u1), unit_c(u1), log2g, log2S, B);
      if (u == ns) {
#pragma unroll
        for (int i = 0; i < kGemvRows; ++i)
#pragma unroll
          for (int q = 0; q < NB; ++q) { acc0[i][q] = accT[i][q]; accT[i][q] = 0.0f; }
      }
      use_slab<NB, GPL, SPL>(A, pj, accT);
      if (u + 1 >= nu) break;
      const int u2 = u + 2 < nu ? u + 2 : nu - 1;
      load_slab<NB, GPL, SPL, SIGN>(jb, unit_r(u2), unit_c(u2), log2g, log2S, A);
      if (u + 1 == ns) {
#pragma unroll
        for (int i = 0; i < kGemvRows; ++i)
#pragma unroll
          for (int q = 0; q < NB; ++q) { acc0[i][q] = accT[i][q]; accT[i][q] = 0.0f; }
      }
      use_slab<NB, GPL, SPL>(B, pj, accT);
    }
    if (nu == ns) {
#pragma unroll
      for (int i = 0; i < kGemvRows; ++i)
#pragma unroll
        for (int q = 0; q < NB; ++q) { acc0[i][q] = accT[i][q]; accT[i][q] = 0.0f; }
    }
  }
#pragma unroll
  for (int i = 0; i < kGemvRows; ++i)
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const float v0 = wave_sum(acc0[i][q]);
      const float v1 = wave_sum(accT[i][q]);
      if (lane == 0) { red[0][wave][i][q] = v0; red[1][wave][i][q] = v1; }
    }
  __syncthreads();
  // the first wave of each row block adds its k partials in wave order
  if (part == 0 && lane < 2 * kGemvRows * NB) {
    const int h = lane / (kGemvRows * NB), i = (lane / NB) % kGemvRows, q = lane % NB;
    float v = red[h][wave][i][q];
    for (int w = 1; w < k; ++w) v += red[h][wave + w][i][q];
    const int64_t r = (h ? r0b : r0a) + i;
    if (r < R) jb.y[q * R + r] = v;
  }
}

template <int NB, int GPL, int SPL, bool SIGN>
void launch_t(const GemvBatch& b, hipStream_t stream) {
  hipLaunchKernelGGL((gemv_kernel<NB, GPL, SPL, SIGN>), dim3((unsigned)b.total_tasks), dim3(kBlock),
                     0, stream, b);
}

template <int NB>
void launch_nb(const GemvBatch& b, hipStream_t stream) {
  const int GPL = b.g >= 32 ? 1 : 32 / b.g;
  const int SPL = b.S >= 32 ? 1 : 32 / b.S;
  if (b.S == b.g) {
    if (GPL == 1) return launch_t<NB, 1, 1, true>(b, stream);
    if (GPL == 2) return launch_t<NB, 2, 2, true>(b, stream);
    return launch_t<NB, 4, 4, true>(b, stream);
  }
  // S < g: GPL <= SPL
  if (GPL == 1 && SPL == 1) return launch_t<NB, 1, 1, false>(b, stream);
  if (GPL == 1 && SPL == 2) return launch_t<NB, 1, 2, false>(b, stream);
  if (GPL == 1) return launch_t<NB, 1, 4, false>(b, stream);
  return launch_t<NB, 2, 4, false>(b, stream);
}

}  // namespace

int gemv_split(int64_t C) {
  const int64_t nslab = (C + kGemvSlab - 1) / kGemvSlab;
  return nslab <= 2 ? 1 : (nslab <= 4 ? 2 : 4);
}

int64_t gemv_tasks(int64_t R, int64_t C) {
  const int64_t rows = 2 * (int64_t)(kWavesPerBlock / gemv_split(C)) * kGemvRows;
  return (R + rows - 1) / rows;
}

hipError_t launch_gemv(const GemvBatch& b, hipStream_t stream) {
  if (b.total_tasks <= 0) return hipSuccess;
  switch (b.B) {
    case 1: launch_nb<1>(b, stream); break;
    case 2: launch_nb<2>(b, stream); break;
    case 3: launch_nb<3>(b, stream); break;
    default: launch_nb<4>(b, stream); break;
  }
  return hipGetLastError();
}

}  // namespace aaac
