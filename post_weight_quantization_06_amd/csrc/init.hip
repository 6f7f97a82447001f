// Table initialization (AAAC summary §2 mechanism 4): equally spaced quantiles of the normalized
// weights, T1 half a step above T0, found by an exact radix select, for up to kMaxJobs matrices in
// one set of launches.
//
// u = fl32(w / s) (IEEE division; u = +0 when s = 0) is mapped to an order-preserving 32-bit key
// (flip all bits of negatives, set the sign bit of non-negatives). The 2n target ranks are resolved
// one byte at a time, most significant first: pass 1 histograms the top byte of every key; after
// each pass one workgroup per matrix walks the histogram of every target's current prefix to the
// byte that holds its residual rank; passes 2-4 histogram the next byte of the keys whose prefix is
// one of the (at most 2n) active prefixes. Integer counts make every step exact and order-free.
//
// Workspace: kMaxJobs headers of (hist u64 [32][256] | state), then the keys u32 [N_i] of every
// matrix. The headers sit at fixed offsets, so a workspace reused for other matrices (or another
// count of them) still starts from the zero histograms the previous call left behind.
#include "common.h"

namespace aaac {

namespace {

constexpr int kTargets = 32;
constexpr int kDigits = 256;

struct InitState {
  uint32_t prefix[kTargets];     // resolved high bytes of each target's key
  uint64_t rank[kTargets];       // residual rank inside that prefix
  uint32_t active[kTargets];     // sorted distinct prefixes of the current pass
  uint32_t nactive;
  uint32_t fold;                 // shift of the prefix table's slot hash for the next pass
  uint32_t pad[2];
};

constexpr size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
constexpr size_t kHistBytes = align256(sizeof(unsigned long long) * kTargets * kDigits);
constexpr size_t kHeaderBytes = kHistBytes + align256(sizeof(InitState));
constexpr size_t kHeadersBytes = kMaxJobs * kHeaderBytes;

// One matrix of an init batch.
struct InitJob {
  const uint16_t* W;
  int64_t R, C, N;
  int64_t nslab;                 // 512-column slabs per row
  uint32_t* keys;                // [N]
  unsigned long long* hist;      // [32][256], zero between calls
  InitState* state;
  float* tables;                 // [2][n]
  int64_t task_begin;            // first keys task (kRowsPerTask rows of one slab)
  int64_t chunk_begin;           // first pass chunk (kChunkVecs 16-byte vectors of keys)
};

struct InitBatch {
  InitJob job[kMaxJobs];
  int njobs, g, n;
  int64_t total_tasks, total_chunks;
};

__device__ __forceinline__ uint32_t order_key(float u) {
  const uint32_t b = __float_as_uint(u);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ void flush_hist(const uint32_t* lds, unsigned long long* hist, int bins) {
  for (int i = threadIdx.x; i < bins; i += (int)blockDim.x)
    if (lds[i]) atomicAdd(hist + i, (unsigned long long)lds[i]);
}

}  // namespace

// Keys of all weights (same lane mapping as assign's 8-weight mapping) and the histogram of their
// top byte. A workgroup walks a contiguous range of tasks; its LDS histogram goes to a matrix's
// histogram when the workgroup leaves that matrix.
__global__ __launch_bounds__(kBlock) void init_keys_kernel(InitBatch b) {
  // eight copies of the histogram, by lane & 7: most keys share a few top bytes, and adds to one
  // address from many lanes of an instruction are serialized
  constexpr int kCopies = 8;
  __shared__ uint32_t h[kCopies][kDigits];
  const int tid = threadIdx.x;
#pragma unroll
  for (int c = 0; c < kCopies; ++c) h[c][tid] = 0;
  __syncthreads();
  const int lane = tid & (kWave - 1), wave = tid / kWave, g8 = b.g / kPerLane;
  const int64_t t_end = task_lo(blockIdx.x + 1, b.total_tasks, gridDim.x);
  int cur = -1;
  auto flush = [&](int j) {
    __syncthreads();
    uint32_t tot = 0;
#pragma unroll
    for (int c = 0; c < kCopies; ++c) {
      tot += h[c][tid];
      h[c][tid] = 0;
    }
    if (tot) atomicAdd(b.job[j].hist + tid, (unsigned long long)tot);
    __syncthreads();
  };
  for (int64_t task = task_lo(blockIdx.x, b.total_tasks, gridDim.x); task < t_end; ++task) {
    int j = cur < 0 ? 0 : cur;
    while (j + 1 < b.njobs && task >= b.job[j + 1].task_begin) ++j;
    if (j != cur) {
      if (cur >= 0) flush(cur);
      cur = j;
    }
    const InitJob& jb = b.job[j];
    const int64_t local = task - jb.task_begin;
    const int64_t rb = local / jb.nslab;
    const int slab = (int)(local - rb * jb.nslab);
    const int c0 = slab * kSlab + lane * kPerLane;
    const bool active = c0 < jb.C;
    for (int i = 0; i < kRowsPerWave; ++i) {
      const int64_t r = rb * kRowsPerTask + wave + (int64_t)kWavesPerBlock * i;
      if (r >= jb.R) break;
      const int64_t base = r * jb.C + c0;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (active) v = *reinterpret_cast<const uint4*>(jb.W + base);
      const uint32_t amax = block_max_u32(lane_absmax_bits(v), g8);
      if (!active) continue;
      const float s = __uint_as_float(amax << 16);
      float w[8];
      unpack8(v, w);
      uint32_t k[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float u = s > 0.0f ? w[e] / s : 0.0f;
        if (u == 0.0f) u = 0.0f;            // zero is unsigned
        k[e] = order_key(u);
        atomicAdd(&h[tid & (kCopies - 1)][k[e] >> 24], 1u);
      }
      uint4* dst = reinterpret_cast<uint4*>(jb.keys + base);
      dst[0] = make_uint4(k[0], k[1], k[2], k[3]);
      dst[1] = make_uint4(k[4], k[5], k[6], k[7]);
    }
  }
  if (cur >= 0) flush(cur);
}

// Passes 2-4: histogram of byte `pass` (0-based from the top) of keys whose higher bytes match an
// active prefix of their matrix. The active prefixes (at most 32, sorted) are found through a
// 4096-slot table indexed by slot_of(prefix, fold); a slot holds one prefix, and a slot that would
// need more sends its keys to a binary search of the sorted list. The select kernel picks, per
// matrix and pass, the first fold shift that gives every active prefix a slot of its own, so the
// search is only taken when no candidate does. One workgroup of 1024 threads per CU walks a
// contiguous range of chunks: its fixed work (clearing the histogram rows in use, the prefix
// table, flushing its histogram with global atomics) is paid once per CU and matrix, and each
// thread keeps four 16-byte loads in flight.
constexpr int kPassThreads = 1024;
constexpr int kSlots = 4096;
constexpr int kPassUnroll = 4;
constexpr int64_t kChunkVecs = (int64_t)kPassThreads * kPassUnroll;

// Slot of a prefix: its low 12 bits with its bits from `fold` up xored in. Quotients of two bf16
// values have short mantissas, so the low bits alone would be mostly zero and the keys' slot reads
// would pile onto a few LDS banks; the fold spreads them.
__device__ __forceinline__ uint32_t slot_of(uint32_t pre, uint32_t fold) {
  return (pre ^ (pre >> fold)) & (kSlots - 1);
}
constexpr int kFolds = 8;
__constant__ const uint32_t kFoldShift[kFolds] = {12, 11, 13, 10, 14, 9, 15, 8};

__global__ __launch_bounds__(kPassThreads) void init_pass_kernel(InitBatch b, int pass) {
  __shared__ uint32_t h[kTargets * kDigits];
  __shared__ uint32_t act[kTargets];
  // slot entry: (prefix, position in the list); position -1 = no prefix, -2 = several prefixes
  __shared__ uint2 slot[kSlots];
  __shared__ uint32_t cnt[kSlots];
  __shared__ uint32_t nact, fold_s;
  const int tid = threadIdx.x;
  const int pshift = 32 - 8 * pass;       // prefix = key >> pshift
  const int dshift = 24 - 8 * pass;       // digit = (key >> dshift) & 255
  const int64_t c_end = task_lo(blockIdx.x + 1, b.total_chunks, gridDim.x);
  int cur = -1;
  int na = 0;
  uint32_t fold = kFoldShift[0];
  for (int64_t chunk = task_lo(blockIdx.x, b.total_chunks, gridDim.x); chunk < c_end; ++chunk) {
    int j = cur < 0 ? 0 : cur;
    while (j + 1 < b.njobs && chunk >= b.job[j + 1].chunk_begin) ++j;
    if (j != cur) {
      if (cur >= 0) {
        __syncthreads();
        flush_hist(h, b.job[cur].hist, na * kDigits);
      }
      // this matrix's active prefixes and their slots
      __syncthreads();
      if (tid < kTargets) act[tid] = b.job[j].state->active[tid];
      if (tid == 0) {
        nact = b.job[j].state->nactive;
        fold_s = b.job[j].state->fold;
      }
      for (int i = tid; i < kSlots; i += kPassThreads) {
        slot[i] = make_uint2(0u, (uint32_t)-1);
        cnt[i] = 0u;
      }
      __syncthreads();
      na = (int)nact;
      fold = fold_s;
      for (int i = tid; i < na * kDigits; i += kPassThreads) h[i] = 0;   // the rows in use
      if (tid < na) atomicAdd(&cnt[slot_of(act[tid], fold)], 1u);
      __syncthreads();
      if (tid < na) {
        const uint32_t sl = slot_of(act[tid], fold);
        slot[sl] = cnt[sl] == 1u ? make_uint2(act[tid], (uint32_t)tid)
                                 : make_uint2(0u, (uint32_t)-2);
      }
      __syncthreads();
      cur = j;
    }
    const InitJob& jb = b.job[j];
    const int64_t n4 = jb.N / 4;
    const uint4* k4 = reinterpret_cast<const uint4*>(jb.keys);
    const int64_t v0 = (chunk - jb.chunk_begin) * kChunkVecs + tid;
    // four 16-byte loads in flight per thread: unconditional at clamped indices, the out-of-range
    // ones then ignored
    uint4 qs[kPassUnroll];
#pragma unroll
    for (int u = 0; u < kPassUnroll; ++u) {
      const int64_t i = v0 + (int64_t)u * kPassThreads;
      qs[u] = k4[i < n4 ? i : n4 - 1];
    }
#pragma unroll
    for (int u = 0; u < kPassUnroll; ++u) {
      if (v0 + (int64_t)u * kPassThreads >= n4) break;
      const uint32_t kk[4] = {qs[u].x, qs[u].y, qs[u].z, qs[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t pre = kk[e] >> pshift;
        const uint2 en = slot[slot_of(pre, fold)];
        const int i0 = (int)en.y;
        int hit = (i0 >= 0 && en.x == pre) ? i0 : -1;
        if (i0 == -2) {
          int lo = 0, hi = na;               // first active prefix >= pre
          while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (act[mid] < pre) lo = mid + 1; else hi = mid;
          }
          if (lo < na && act[lo] == pre) hit = lo;
        }
        if (hit >= 0) atomicAdd(&h[hit * kDigits + ((kk[e] >> dshift) & 255u)], 1u);
      }
    }
  }
  if (cur >= 0) {
    __syncthreads();
    flush_hist(h, b.job[cur].hist, na * kDigits);
  }
}

// One workgroup of 1024 threads per matrix (a target or two per wave): move every target one byte
// down, rebuild the active prefix list, clear the histogram rows used; after the last pass write
// the tables. The rows in use are first copied to LDS (one coalesced read per thread and row) so
// that each target walks its row there.
constexpr int kSelectThreads = 1024;
__global__ __launch_bounds__(kSelectThreads) void init_select_kernel(InitBatch b, int pass) {
  const InitJob& jb = b.job[blockIdx.x];
  const int64_t N = jb.N;
  const int n = b.n;
  InitState* const state = jb.state;
  unsigned long long* const hist = jb.hist;
  float* const tables = jb.tables;
  const int tid = threadIdx.x;
  const int nt = 2 * n;
  constexpr int kWaves = kSelectThreads / kWave;
  __shared__ uint32_t newp[kTargets];
  __shared__ unsigned long long hl[kTargets * kDigits];
  __shared__ uint32_t first[kTargets];
  if (pass == 0 && tid < nt) {
    // target ranks of reading: T0[j] at floor((2j+1) N / 2n), T1[j] at min(N-1, floor((j+1) N / n))
    const int j = tid % n;
    uint64_t r;
    // N < 2^40, so (2j + 1) N < 2^45 fits in 64 bits
    if (tid < n) {
      r = (uint64_t)(2 * j + 1) * (uint64_t)N / (uint64_t)(2 * n);
    } else {
      r = (uint64_t)(j + 1) * (uint64_t)N / (uint64_t)n;
      if (r > (uint64_t)(N - 1)) r = (uint64_t)(N - 1);
    }
    state->prefix[tid] = 0;
    state->rank[tid] = r;
  }
  __shared__ uint32_t act_s[kTargets], pre_s[kTargets];
  __shared__ uint64_t rank_s[kTargets];
  __shared__ int rows_s;
  if (tid == 0) rows_s = pass == 0 ? 1 : (int)state->nactive;
  if (tid < kTargets) {
    act_s[tid] = state->active[tid];
    pre_s[tid] = state->prefix[tid];
    rank_s[tid] = state->rank[tid];
  }
  __syncthreads();
  const int rows = rows_s;
  // the rows in use and the (zero) row after them, read by a target without a row of its own,
  // which the construction of the active list rules out
  const int copy = rows < kTargets ? rows + 1 : kTargets;
  {
    // thread t reads digit t & 255 of rows t / 256, t / 256 + 4, ...: all its loads before any
    // store
    constexpr int kPer = kTargets * kDigits / kSelectThreads;
    unsigned long long v[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int i = tid + k * kSelectThreads;
      v[k] = i < copy * kDigits ? hist[i] : 0ull;
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int i = tid + k * kSelectThreads;
      if (i < copy * kDigits) hl[i] = v[k];
    }
  }
  __syncthreads();
  {
    // wave w resolves targets w and w + 16: lane l holds the count of digits 4l .. 4l + 3 of the
    // target's row, an inclusive scan over the wave finds the lane whose digits hold the rank,
    // and that lane walks its four digits
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    for (int t = wave; t < nt; t += kWaves) {
      const uint32_t pre = pre_s[t];
      int slot = 0;
      if (pass > 0) {
        // the row of this target's prefix: one compare per lane, first match
        const unsigned long long m = __ballot(lane < rows && act_s[lane & (kTargets - 1)] == pre);
        slot = m ? __builtin_ctzll(m) : copy - 1;
      }
      const uint64_t rank = rank_s[t];
      const unsigned long long* row = hl + slot * kDigits + 4 * lane;
      const uint64_t c0 = row[0], c1 = row[1], c2 = row[2], c3 = row[3];
      const uint64_t mine = c0 + c1 + c2 + c3;
      uint64_t incl = mine;
#pragma unroll
      for (int d = 1; d < kWave; d <<= 1) {
        const uint64_t other = (uint64_t)__shfl_up((unsigned long long)incl, d);
        if (lane >= d) incl += other;
      }
      const uint64_t excl = incl - mine;
      // the first lane whose inclusive count exceeds the rank (the last lane if none does)
      const unsigned long long hit = __ballot(rank < incl);
      const int owner = hit ? __builtin_ctzll(hit) : kWave - 1;
      if (lane == owner) {
        uint64_t cum = excl;
        int d = 4 * lane;
        if (rank >= cum + c0 && d < kDigits - 1) { cum += c0; ++d;
          if (rank >= cum + c1 && d < kDigits - 1) { cum += c1; ++d;
            if (rank >= cum + c2 && d < kDigits - 1) { cum += c2; ++d; } } }
        newp[t] = (pre << 8) | (uint32_t)d;
        state->rank[t] = rank - cum;
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < rows * kDigits; i += kSelectThreads) hist[i] = 0ull;
  if (tid < nt) {
    state->prefix[tid] = newp[tid];
    // first occurrence of this prefix among the targets
    uint32_t f = 1;
    for (int t = 0; t < tid; ++t) f = (newp[t] == newp[tid]) ? 0u : f;
    first[tid] = f;
  }
  __syncthreads();
  if (tid < nt && first[tid]) {
    // position in the sorted list of distinct prefixes
    int pos = 0;
    for (int t = 0; t < nt; ++t) pos += (first[t] && newp[t] < newp[tid]) ? 1 : 0;
    state->active[pos] = newp[tid];
  }
  if (tid == 0) {
    uint32_t m = 0;
    for (int t = 0; t < nt; ++t) m += first[t];
    state->nactive = m;
  }
  if (pass == 3) {
    if (tid < nt) tables[tid] = key_value(newp[tid]);
    return;
  }
  // the slot hash of the next pass: wave w tries fold candidate w; lane t holds target t's slot
  // (or a value no slot takes when t repeats an earlier target's prefix) and looks for an equal
  // slot on a lower lane
  __shared__ uint32_t fold_ok[kFolds];
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  if (wave < kFolds) {
    const uint32_t f = kFoldShift[wave];
    const uint32_t mine =
        (lane < nt && first[lane]) ? slot_of(newp[lane], f) : (uint32_t)(kSlots + lane);
    bool clash = false;
    for (int t = 0; t < kTargets; ++t) {
      const uint32_t other = (uint32_t)__shfl((int)mine, t);
      clash = clash || (t < lane && other == mine);
    }
    const unsigned long long any = __ballot(clash);
    if (lane == 0) fold_ok[wave] = any ? 0u : 1u;
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t f = kFoldShift[0];
    for (int c = kFolds - 1; c >= 0; --c) f = fold_ok[c] ? kFoldShift[c] : f;
    state->fold = f;
  }
}

size_t init_workspace_bytes(int count, const int64_t* R, const int64_t* C) {
  size_t bytes = kHeadersBytes;
  for (int i = 0; i < count; ++i) bytes += align256((size_t)R[i] * (size_t)C[i] * 4);
  return bytes;
}

hipError_t launch_init(int count, const uint16_t* const* W, const int64_t* R, const int64_t* C,
                       int g, int n, float* const* tables, void* ws, hipStream_t stream) {
  InitBatch b{};
  b.njobs = count;
  b.g = g;
  b.n = n;
  char* const base = static_cast<char*>(ws);
  char* keys = base + kHeadersBytes;
  int64_t tb = 0, cb = 0;
  for (int i = 0; i < count; ++i) {
    InitJob& j = b.job[i];
    const MatrixGeom geom = make_geom(R[i], C[i], tb);
    j.W = W[i];
    j.R = R[i];
    j.C = C[i];
    j.N = R[i] * C[i];
    j.nslab = geom.nslab;
    j.hist = reinterpret_cast<unsigned long long*>(base + (size_t)i * kHeaderBytes);
    j.state = reinterpret_cast<InitState*>(base + (size_t)i * kHeaderBytes + kHistBytes);
    j.keys = reinterpret_cast<uint32_t*>(keys);
    keys += align256((size_t)j.N * 4);
    j.tables = tables[i];
    j.task_begin = tb;
    tb += geom.ntasks;
    j.chunk_begin = cb;
    cb += (j.N / 4 + kChunkVecs - 1) / kChunkVecs;
  }
  b.total_tasks = tb;
  b.total_chunks = cb;
  const int64_t cus = device_cu_count();
  const int grid1 = (int)(tb < cus * 4 ? tb : cus * 4);
  hipLaunchKernelGGL(init_keys_kernel, dim3(grid1), dim3(kBlock), 0, stream, b);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(init_select_kernel, dim3(count), dim3(kSelectThreads), 0, stream, b, 0);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int grid = (int)(cb < cus ? cb : cus);
  for (int pass = 1; pass < 4; ++pass) {
    hipLaunchKernelGGL(init_pass_kernel, dim3(grid), dim3(kPassThreads), 0, stream, b, pass);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(init_select_kernel, dim3(count), dim3(kSelectThreads), 0, stream, b, pass);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace aaac
