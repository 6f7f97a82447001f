// Table initialization (AAAC summary §2 mechanism 4): equally spaced quantiles of the normalized
// weights, T1 half a step above T0, found by an exact radix select, for up to kMaxJobs matrices in
// one set of launches.
//
// u = fl32(w / s) (IEEE division; u = +0 when s = 0) is mapped to an order-preserving 32-bit key
// (flip all bits of negatives, set the sign bit of non-negatives). The 2n target ranks are resolved
// in three digits, most significant first: 12 bits, then 10, then 10. The keys kernel histograms
// the top 12 bits of every key; after each histogram one workgroup per matrix walks the histogram
// row of every target's current prefix to the digit that holds its residual rank; two passes then
// histogram the next 10 bits of the keys whose prefix is one of the (at most 2n) active prefixes.
// Integer counts make every step exact and order-free.
//
// Workspace: kMaxJobs headers of (hist u64 [32][1024] | state), then the keys u32 [N_i] of every
// matrix. The headers sit at fixed offsets, so a workspace reused for other matrices (or another
// count of them) still starts from the zero histograms the previous call left behind.
#include "common.h"

namespace aaac {

namespace {

constexpr int kTargets = 32;
// digits: step 0 (the keys kernel) takes the top kTopBits of a key, steps 1 and 2 (the passes)
// kLowBits each
constexpr int kTopBits = 12;
constexpr int kTopDigits = 1 << kTopBits;
constexpr int kLowBits = 10;
constexpr int kLowDigits = 1 << kLowBits;
constexpr int kSteps = 3;
constexpr int kHistBins = kTargets * kLowDigits;      // [target row][digit]; step 0 uses row 0..3
static_assert(kTopBits + (kSteps - 1) * kLowBits == 32, "the digits cover the key");
static_assert(kTopDigits <= kHistBins, "the top digit's histogram fits the rows");

struct InitState {
  uint32_t prefix[kTargets];     // resolved high bytes of each target's key
  uint64_t rank[kTargets];       // residual rank inside that prefix
  uint32_t active[kTargets];     // sorted distinct prefixes of the next step
  uint32_t nactive;
  uint32_t hash;                 // multiplier of the prefix table's slot hash for the next step
  uint32_t pad[2];
};

constexpr size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
constexpr size_t kHistBytes = align256(sizeof(unsigned long long) * kHistBins);
constexpr size_t kHeaderBytes = kHistBytes + align256(sizeof(InitState));
constexpr size_t kHeadersBytes = kMaxJobs * kHeaderBytes;

// One matrix of an init batch.
struct InitJob {
  const uint16_t* W;
  int64_t R, C, N;
  int64_t nslab;                 // 512-column slabs per row
  uint32_t* keys;                // [N]
  unsigned long long* hist;      // [32][1024], zero between calls
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
// top 12 bits. A workgroup walks a contiguous range of tasks; its LDS histogram goes to a matrix's
// histogram when the workgroup leaves that matrix.
__global__ __launch_bounds__(kBlock) void init_keys_kernel(InitBatch b) {
  // two copies of the histogram, by lane parity: the busiest bins hold a few percent of the keys,
  // and adds to one address from several lanes of an instruction are serialized
  constexpr int kCopies = 2;
  __shared__ uint32_t h[kCopies][kTopDigits];
  const int tid = threadIdx.x;
  for (int i = tid; i < kCopies * kTopDigits; i += kBlock) (&h[0][0])[i] = 0;
  __syncthreads();
  const int lane = tid & (kWave - 1), wave = tid / kWave, g8 = b.g / kPerLane;
  const int64_t t_end = task_lo(blockIdx.x + 1, b.total_tasks, gridDim.x);
  int cur = -1;
  auto flush = [&](int j) {
    __syncthreads();
    for (int i = tid; i < kTopDigits; i += kBlock) {
      uint32_t tot = 0;
#pragma unroll
      for (int c = 0; c < kCopies; ++c) {
        tot += h[c][i];
        h[c][i] = 0;
      }
      if (tot) atomicAdd(b.job[j].hist + i, (unsigned long long)tot);
    }
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
    // all rows of the task loaded before any is used (clamped in-bounds rows; a lane past the
    // last column holds zeros)
    uint4 vr[kRowsPerWave];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      int64_t r = rb * kRowsPerTask + wave + (int64_t)kWavesPerBlock * i;
      r = r < jb.R ? r : jb.R - 1;
      vr[i] = active ? *reinterpret_cast<const uint4*>(jb.W + r * jb.C + c0)
                     : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      const int64_t r = rb * kRowsPerTask + wave + (int64_t)kWavesPerBlock * i;
      if (r >= jb.R) break;                              // the same for the whole wave
      const int64_t base = r * jb.C + c0;
      const uint4 v = vr[i];
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
        atomicAdd(&h[tid & (kCopies - 1)][k[e] >> (32 - kTopBits)], 1u);
      }
      uint4* dst = reinterpret_cast<uint4*>(jb.keys + base);
      dst[0] = make_uint4(k[0], k[1], k[2], k[3]);
      dst[1] = make_uint4(k[4], k[5], k[6], k[7]);
    }
  }
  if (cur >= 0) flush(cur);
}

// Steps 1 and 2: histogram of the next 10 bits of the keys whose higher bits match an active prefix
// of their matrix. The active prefixes (at most 32, sorted) are found through a 2048-slot table
// indexed by slot_of(prefix, hash); a slot holds one prefix, and a slot that would need more sends
// its keys to a binary search of the sorted list. The select kernel picks, per matrix and step,
// the first hash multiplier that gives every active prefix a slot of its own, so the search is
// only taken when no candidate does. One workgroup of 1024 threads per CU walks a contiguous range
// of chunks: its fixed work (clearing the histogram rows in use, the prefix table, flushing its
// histogram with global atomics) is paid once per CU and matrix, and each thread keeps four
// 16-byte loads in flight.
constexpr int kPassThreads = 1024;
constexpr int kSlotBits = 11;
constexpr int kSlots = 1 << kSlotBits;
constexpr int kPassUnroll = 4;
constexpr int64_t kChunkVecs = (int64_t)kPassThreads * kPassUnroll;
// slot entry: prefix << 5 | position in the sorted list, or one of two markers (neither equals a
// 22-bit prefix once shifted down by 5)
constexpr uint32_t kSlotEmpty = 0xFFFFFFFFu;
constexpr uint32_t kSlotShared = 0xFFFFFFFEu;
static_assert(kTopBits + kLowBits + 5 <= 32, "a slot entry holds a prefix and a position");

// Slot of a prefix (at most 22 bits): the top 11 bits of the low 32 bits of prefix x hash, a
// 24-bit odd multiplier (one full-rate 24-bit multiply). Quotients of two bf16 values have short
// mantissas, so the prefixes' low bits are mostly zero; the product mixes every bit of the prefix
// into the slot, which also spreads the keys' slot reads over the LDS banks.
__device__ __forceinline__ uint32_t slot_of(uint32_t pre, uint32_t hash) {
  // HIP's __umul24 returns int: the shift must see the product as unsigned
  return static_cast<uint32_t>(__umul24(pre, hash)) >> (32 - kSlotBits);
}
constexpr int kHashes = 8;
__constant__ const uint32_t kHashMul[kHashes] = {0x9E3779u, 0x85EBCBu, 0xC2B2AFu, 0x27D4EBu,
                                                 0x165667u, 0xB55A4Fu, 0x7FEB35u, 0x61C887u};

__global__ __launch_bounds__(kPassThreads) void init_pass_kernel(InitBatch b, int step) {
  __shared__ uint32_t h[kHistBins];
  __shared__ uint32_t act[kTargets];
  __shared__ uint32_t slot[kSlots];
  __shared__ uint32_t cnt[kSlots];
  __shared__ uint32_t nact, hash_s;
  const int tid = threadIdx.x;
  const int pshift = 32 - kTopBits - kLowBits * (step - 1);   // prefix = key >> pshift
  const int dshift = pshift - kLowBits;                        // digit = (key >> dshift) & 1023
  const int64_t c_end = task_lo(blockIdx.x + 1, b.total_chunks, gridDim.x);
  int cur = -1;
  int na = 0;
  uint32_t hash = kHashMul[0];
  for (int64_t chunk = task_lo(blockIdx.x, b.total_chunks, gridDim.x); chunk < c_end; ++chunk) {
    int j = cur < 0 ? 0 : cur;
    while (j + 1 < b.njobs && chunk >= b.job[j + 1].chunk_begin) ++j;
    if (j != cur) {
      if (cur >= 0) {
        __syncthreads();
        flush_hist(h, b.job[cur].hist, na * kLowDigits);
      }
      // this matrix's active prefixes and their slots
      __syncthreads();
      if (tid < kTargets) act[tid] = b.job[j].state->active[tid];
      if (tid == 0) {
        nact = b.job[j].state->nactive;
        hash_s = b.job[j].state->hash;
      }
      for (int i = tid; i < kSlots; i += kPassThreads) {
        slot[i] = kSlotEmpty;
        cnt[i] = 0u;
      }
      __syncthreads();
      na = (int)nact;
      hash = hash_s;
      for (int i = tid; i < na * kLowDigits; i += kPassThreads) h[i] = 0;   // the rows in use
      if (tid < na) atomicAdd(&cnt[slot_of(act[tid], hash)], 1u);
      __syncthreads();
      if (tid < na) {
        const uint32_t sl = slot_of(act[tid], hash);
        slot[sl] = cnt[sl] == 1u ? (act[tid] << 5) | (uint32_t)tid : kSlotShared;
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
    // all 16 slot reads, then the hits, then all 16 adds: a search between them would make every
    // key wait for the LDS operations in flight, the previous key's add included, and adds to
    // the one bin of u = 1 or u = -1 are slow when every group has its maximum there
    constexpr int kKeys = 4 * kPassUnroll;
    uint32_t kk[kKeys], en[kKeys];
#pragma unroll
    for (int u = 0; u < kPassUnroll; ++u) {
      kk[4 * u] = qs[u].x;
      kk[4 * u + 1] = qs[u].y;
      kk[4 * u + 2] = qs[u].z;
      kk[4 * u + 3] = qs[u].w;
    }
#pragma unroll
    for (int i = 0; i < kKeys; ++i) en[i] = slot[slot_of(kk[i] >> pshift, hash)];
    int hit[kKeys];
    bool shared = false;
#pragma unroll
    for (int i = 0; i < kKeys; ++i) {
      const uint32_t pre = kk[i] >> pshift;
      const bool valid = v0 + (int64_t)(i / 4) * kPassThreads < n4;
      hit[i] = (valid && (en[i] >> 5) == pre) ? (int)(en[i] & 31u) : -1;
      shared = shared || (valid && en[i] == kSlotShared);
    }
    if (__ballot(shared)) {
      for (int i = 0; i < kKeys; ++i) {
        const uint32_t pre = kk[i] >> pshift;
        const bool valid = v0 + (int64_t)(i / 4) * kPassThreads < n4;
        if (valid && en[i] == kSlotShared) {
          int lo = 0, hi = na;               // first active prefix >= pre
          while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (act[mid] < pre) lo = mid + 1; else hi = mid;
          }
          if (lo < na && act[lo] == pre) hit[i] = lo;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kKeys; ++i)
      if (hit[i] >= 0)
        atomicAdd(&h[hit[i] * kLowDigits + ((kk[i] >> dshift) & (kLowDigits - 1))], 1u);
  }
  if (cur >= 0) {
    __syncthreads();
    flush_hist(h, b.job[cur].hist, na * kLowDigits);
  }
}

// One workgroup of 1024 threads per matrix (a target or two per wave): move every target one digit
// down, rebuild the active prefix list, clear the histogram rows used; after the last step write
// the tables. A wave finds its target's digit in two steps over the row, which sits in L2 after
// the histogram kernel's atomics: lane l first sums digits [l P, (l + 1) P) (P = 64 or 16), an
// inclusive scan over the wave and a ballot find the lane whose block holds the rank, then lane j
// reads digit j of that block and a second scan and ballot find the digit.
constexpr int kSelectThreads = 1024;

struct DigitPick {
  uint32_t digit;   // the digit whose count range holds the rank
  uint64_t rest;    // the rank's residual inside that digit
};

__device__ __forceinline__ uint64_t wave_incl_scan(uint64_t v, int lane) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const uint64_t other = (uint64_t)__shfl_up((unsigned long long)v, d);
    if (lane >= d) v += other;
  }
  return v;
}

// A histogram row staged in LDS: one u64 of padding after every 32 digits, so that lanes reading
// blocks of 16 or 64 consecutive digits start on different banks.
__device__ __forceinline__ int padded(int d) { return d + (d >> 5); }
constexpr int kPaddedLow = kLowDigits + kLowDigits / 32;
constexpr int kPaddedTop = kTopDigits + kTopDigits / 32;

// The digit of a staged histogram row (kPer * 64 bins) that holds `rank`, the same on every lane.
template <int kPer>
__device__ __forceinline__ DigitPick pick_digit(const unsigned long long* row, uint64_t rank,
                                                int lane) {
  // first: lane l sums digits [l kPer, (l + 1) kPer)
  uint64_t mine = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) mine += row[padded(lane * kPer + k)];
  const uint64_t incl = wave_incl_scan(mine, lane);
  // the first lane whose inclusive count exceeds the rank (the last lane if none does)
  const unsigned long long hit = __ballot(rank < incl);
  const int owner = hit ? __builtin_ctzll(hit) : kWave - 1;
  const uint64_t base = (uint64_t)__shfl((unsigned long long)(incl - mine), owner);
  // then: lane j < kPer takes digit j of the owner's block
  const uint64_t c = lane < kPer ? (uint64_t)row[padded(owner * kPer + lane)] : 0ull;
  const uint64_t incl2 = base + wave_incl_scan(c, lane);
  const unsigned long long hit2 = __ballot(lane < kPer && rank < incl2);
  const int dl = hit2 ? __builtin_ctzll(hit2) : kPer - 1;
  const uint64_t below = (uint64_t)__shfl((unsigned long long)(incl2 - c), dl);
  return DigitPick{(uint32_t)(owner * kPer + dl), rank - below};
}

__global__ __launch_bounds__(kSelectThreads) void init_select_kernel(InitBatch b, int step) {
  const InitJob& jb = b.job[blockIdx.x];
  const int64_t N = jb.N;
  const int n = b.n;
  InitState* const state = jb.state;
  unsigned long long* const hist = jb.hist;
  float* const tables = jb.tables;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int nt = 2 * n;
  constexpr int kWaves = kSelectThreads / kWave;
  __shared__ uint32_t newp[kTargets];
  __shared__ uint32_t first[kTargets];
  if (step == 0 && tid < nt) {
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
  if (tid == 0) rows_s = step == 0 ? 1 : (int)state->nactive;
  if (tid < kTargets) {
    act_s[tid] = state->active[tid];
    pre_s[tid] = state->prefix[tid];
    rank_s[tid] = state->rank[tid];
  }
  __syncthreads();
  const int rows = rows_s;
  const int dbits = step == 0 ? kTopBits : kLowBits;
  // staged rows: the top digit's one row for every wave, or one row per wave
  static_assert(kWaves * kPaddedLow >= kPaddedTop, "the top digit's row fits the staging area");
  __shared__ unsigned long long rowbuf[kWaves * kPaddedLow];
  if (step == 0) {
    for (int i = tid; i < kTopDigits; i += kSelectThreads) rowbuf[padded(i)] = hist[i];
  }
  __syncthreads();
  // every wave runs the same number of rounds, so the block barriers match
  static_assert(kTargets % kWaves == 0, "targets per wave");
  for (int r = 0; r < kTargets / kWaves; ++r) {
    const int t = wave + r * kWaves;
    const bool mine = t < nt;
    const uint32_t pre = pre_s[t];
    unsigned long long* const wrow = rowbuf + wave * kPaddedLow;
    if (step > 0 && mine) {
      // the row of this target's prefix: one compare per lane, first match (the construction of
      // the active list gives every target one; the fallback is a zero row or the last row)
      const unsigned long long m = __ballot(lane < rows && act_s[lane & (kTargets - 1)] == pre);
      const int row = m ? __builtin_ctzll(m) : (rows < kTargets ? rows : kTargets - 1);
      const unsigned long long* const hrow = hist + (size_t)row * kLowDigits;
#pragma unroll
      for (int k = 0; k < kLowDigits / kWave; ++k)
        wrow[padded(k * kWave + lane)] = hrow[k * kWave + lane];
    }
    __syncthreads();
    if (mine) {
      const DigitPick pk = step == 0 ? pick_digit<kTopDigits / kWave>(rowbuf, rank_s[t], lane)
                                     : pick_digit<kLowDigits / kWave>(wrow, rank_s[t], lane);
      if (lane == 0) {
        newp[t] = (pre << dbits) | pk.digit;
        state->rank[t] = pk.rest;
      }
    }
    __syncthreads();
  }
  // clear what this step's histogram used: the top digit's 4096 bins, or the rows in use
  const int used = step == 0 ? kTopDigits : rows * kLowDigits;
  for (int i = tid; i < used; i += kSelectThreads) hist[i] = 0ull;
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
  if (step == kSteps - 1) {
    if (tid < nt) tables[tid] = key_value(newp[tid]);
    return;
  }
  // the slot hash of the next step: wave w tries multiplier w; lane t holds target t's slot (or a
  // value no slot takes when t repeats an earlier target's prefix) and looks for an equal slot on
  // a lower lane
  __shared__ uint32_t hash_ok[kHashes];
  if (wave < kHashes) {
    const uint32_t f = kHashMul[wave];
    const uint32_t mine =
        (lane < nt && first[lane]) ? slot_of(newp[lane], f) : (uint32_t)(kSlots + lane);
    bool clash = false;
    for (int t = 0; t < kTargets; ++t) {
      const uint32_t other = (uint32_t)__shfl((int)mine, t);
      clash = clash || (t < lane && other == mine);
    }
    const unsigned long long any = __ballot(clash);
    if (lane == 0) hash_ok[wave] = any ? 0u : 1u;
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t f = kHashMul[0];
    for (int c = kHashes - 1; c >= 0; --c) f = hash_ok[c] ? kHashMul[c] : f;
    state->hash = f;
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
  for (int step = 1; step < kSteps; ++step) {
    hipLaunchKernelGGL(init_pass_kernel, dim3(grid), dim3(kPassThreads), 0, stream, b, step);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(init_select_kernel, dim3(count), dim3(kSelectThreads), 0, stream, b, step);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace aaac
