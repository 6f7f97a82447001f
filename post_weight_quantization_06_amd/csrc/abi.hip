// C ABI of the quantizer (declared in include/aaac.h): argument checks, workspace layout and
// kernel launches on the caller's stream. Nothing here allocates, frees or synchronizes.
#include <stdarg.h>
#include <stdio.h>

#include <atomic>

#include "aaac.h"
#include "common.h"

namespace aaac {

int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

}  // namespace aaac

namespace {

using namespace aaac;

thread_local char g_err[512];

aaac_status fail(aaac_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

aaac_status ok() {
  g_err[0] = '\0';
  return AAAC_OK;
}

aaac_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(AAAC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Shape rules shared by the matrix calls. need_S: the call uses the selection group.
aaac_status check_shape(int64_t R, int64_t C, int g, int S, int n, bool need_S, const char* who) {
  if (R < 1 || C < 8 || C % 8 != 0 || C >= ((int64_t)1 << 31))
    return fail(AAAC_ERR_UNSUPPORTED_SHAPE, "%s: R=%lld C=%lld (need R >= 1, C >= 8, C %% 8 == 0)",
                who, (long long)R, (long long)C);
  if (R > ((((int64_t)1 << 40) - 1) / C))
    return fail(AAAC_ERR_UNSUPPORTED_SHAPE, "%s: R*C must stay below 2^40", who);
  if (!pow2(g) || g < 8 || g > 512 || C % g != 0)
    return fail(AAAC_ERR_UNSUPPORTED_SHAPE, "%s: g=%d (need a power of two in [8, 512] dividing C)",
                who, g);
  if (need_S && (!pow2(S) || S < 8 || S > g))
    return fail(AAAC_ERR_UNSUPPORTED_SHAPE, "%s: S=%d (need a power of two in [8, g])", who, S);
  if (n < 2 || n > 16)
    return fail(AAAC_ERR_UNSUPPORTED_SHAPE, "%s: n=%d (need 2 <= n <= 16)", who, n);
  return AAAC_OK;
}

// refine workspace: job counters (256 bytes), then fp64 partials [count][kPartVals][kMaxRefineBlocks]
size_t refine_ws_bytes(int count) {
  return 256 + (size_t)count * kPartVals * kMaxRefineBlocks * sizeof(double);
}

aaac_status check_batch(int count, const uint16_t* const* W, const int64_t* R, const int64_t* C,
                        int g, int S, int n, const char* who) {
  if (count < 1 || count > AAAC_MAX_BATCH)
    return fail(AAAC_ERR_INVALID_ARG, "%s: count=%d (need 1..%d)", who, count, AAAC_MAX_BATCH);
  if (!W || !R || !C) return fail(AAAC_ERR_INVALID_ARG, "%s: null array", who);
  for (int i = 0; i < count; ++i) {
    aaac_status st = check_shape(R[i], C[i], g, S, n, true, who);
    if (st != AAAC_OK) return st;
    if (!W[i] || !aligned(W[i], 16))
      return fail(AAAC_ERR_INVALID_ARG, "%s: W[%d] null or not 16-byte aligned", who, i);
  }
  return AAAC_OK;
}

// assign workspace (only with error totals): job counters (256 bytes), then fp64 partials
// [count][kMaxAssignBlocks]
size_t assign_ws_bytes(int count) {
  return 256 + (size_t)count * kMaxAssignBlocks * sizeof(double);
}

aaac_status check_assign_args(int count, const uint16_t* const* W, const int64_t* R,
                              const int64_t* C, int g, int S, int n, const float* const* I,
                              const float* const* tables, uint8_t* const* codes,
                              uint8_t* const* sel, const char* who) {
  aaac_status st = check_batch(count, W, R, C, g, S, n, who);
  if (st != AAAC_OK) return st;
  if (!I || !tables || !codes || !sel) return fail(AAAC_ERR_INVALID_ARG, "%s: null array", who);
  for (int i = 0; i < count; ++i) {
    if (!I[i] || !aligned(I[i], 16) || !tables[i] || !aligned(tables[i], 4) || !codes[i] ||
        !aligned(codes[i], 16) || !sel[i])
      return fail(AAAC_ERR_INVALID_ARG,
                  "%s: matrix %d: I, tables, codes or sel null or misaligned (I and codes need 16 "
                  "bytes)", who, i);
  }
  return AAAC_OK;
}

// An assign batch in the 8-weight task numbering (the launcher renumbers for the wide mapping).
void build_assign_batch(AssignBatch& b, int count, const uint16_t* const* W, const int64_t* R,
                        const int64_t* C, int g, int S, int n, const float* const* I,
                        const float* const* tables, uint8_t* const* codes, uint8_t* const* sel) {
  b.njobs = count;
  b.g = g;
  b.S = S;
  b.n = n;
  int64_t tb = 0;
  for (int i = 0; i < count; ++i) {
    AssignJob& j = b.job[i];
    j.geom = make_geom(R[i], C[i], tb);
    tb += j.geom.ntasks;
    j.W = W[i];
    j.I = I[i];
    j.tables = tables[i];
    j.codes = reinterpret_cast<uint32_t*>(codes[i]);
    j.sel = sel[i];
  }
  b.total_tasks = tb;
}

aaac_status do_assign(int count, const uint16_t* const* W, const int64_t* R, const int64_t* C,
                      int g, int S, int n, const float* const* I, const float* const* tables,
                      uint8_t* const* codes, uint8_t* const* sel, double* err, double* err_total,
                      void* ws, size_t ws_bytes, void* stream, const char* who) {
  aaac_status st = check_assign_args(count, W, R, C, g, S, n, I, tables, codes, sel, who);
  if (st != AAAC_OK) return st;
  if (err && !aligned(err, 8)) return fail(AAAC_ERR_INVALID_ARG, "%s: err misaligned", who);
  if (err_total) {
    if (!aligned(err_total, 8))
      return fail(AAAC_ERR_INVALID_ARG, "%s: err_total misaligned", who);
    if (!ws || !aligned(ws, 256))
      return fail(AAAC_ERR_INVALID_ARG, "%s: ws null or not 256-byte aligned (needed with err_total)",
                  who);
    if (ws_bytes < assign_ws_bytes(count))
      return fail(AAAC_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu < %zu bytes", who, ws_bytes,
                  assign_ws_bytes(count));
  }
  AssignBatch b{};
  build_assign_batch(b, count, W, R, C, g, S, n, I, tables, codes, sel);
  for (int i = 0; i < count; ++i) {
    b.job[i].err = err;
    b.job[i].err_total = err_total ? err_total + i : nullptr;
  }
  if (err_total) {
    b.totals = 1;
    b.counters = static_cast<uint32_t*>(ws);
    b.partials = reinterpret_cast<double*>(static_cast<char*>(ws) + 256);
  }
  return hip_status(launch_assign(b, err != nullptr, static_cast<hipStream_t>(stream)), who);
}

// Batch description shared by refine and the fused assign + accumulate: task geometry, grid,
// and the workgroup range that meets each job (its slots in the partials).
void build_refine_batch(RefineBatch& b, int count, const uint16_t* const* W, const int64_t* R,
                        const int64_t* C, int g, int S, int n, const float* const* I, int flags,
                        void* ws) {
  b.njobs = count;
  b.g = g;
  b.S = S;
  b.n = n;
  b.flags = flags;
  int64_t tb = 0;
  for (int i = 0; i < count; ++i) {
    RefineJob& j = b.job[i];
    j.geom = refine_geom(R[i], C[i], tb, S);
    tb += j.geom.ntasks;
    j.W = W[i];
    j.I = I[i];
  }
  b.total_tasks = tb;
  int64_t nb = refine_grid(tb);
  if (nb > kMaxRefineBlocks) nb = kMaxRefineBlocks;
  b.nblocks = (int32_t)nb;
  // workgroup b owns tasks [task_lo(b), task_lo(b + 1)); record which workgroups meet each job
  b.slots = job_slots(b.job, count, tb, nb);
  b.counters = static_cast<uint32_t*>(ws);
  b.partials = reinterpret_cast<double*>(static_cast<char*>(ws) + 256);
}

aaac_status check_refine_ws(int count, void* ws, size_t ws_bytes, const char* who) {
  const size_t need = refine_ws_bytes(count);
  if (!ws || !aligned(ws, 256)) return fail(AAAC_ERR_INVALID_ARG, "%s: ws null or not 256-byte aligned", who);
  if (ws_bytes < need)
    return fail(AAAC_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu < %zu bytes", who, ws_bytes, need);
  return AAAC_OK;
}

// ------------------------------------------------------------------------------------------------
// Fixed device scratch for aaac_refine_batch_noalloc: the refine workspace of a full batch (job
// counters, then per-workgroup partials), one copy per GPU, alive until the process ends. Host
// code reaches it only through the address hipGetSymbolAddress returns for the current device,
// taken once per device on the first call there.
// ------------------------------------------------------------------------------------------------
constexpr size_t kScratchBytes = 256 + (size_t)kMaxJobs * kPartVals * kMaxRefineBlocks * sizeof(double);

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// The scratch address on the current device, or nullptr (and a message) on failure.
void* scratch_on_current_device(const char* who, aaac_status* st) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *st = fail(AAAC_ERR_HIP, "%s: hipGetDevice: %s", who, hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *st = fail(AAAC_ERR_INVALID_ARG, "%s: device %d beyond the %d this library serves", who, dev,
               kMaxDevices);
    return nullptr;
  }
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p) {
    *st = fail(AAAC_ERR_HIP, "%s: hipGetSymbolAddress(scratch): %s", who, hipGetErrorString(e));
    return nullptr;
  }
  g_scratch_ptr[dev].store(p, std::memory_order_release);
  return p;
}

// Clears n 32-bit words (a kernel rather than a memset, so that the call can be captured in a
// graph).
__global__ void clear_words_kernel(uint32_t* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

// Every argument of a refine call except the workspace.
aaac_status check_refine_args(int count, const uint16_t* const* W, const int64_t* R,
                              const int64_t* C, int g, int S, int n, const float* const* I,
                              const uint8_t* const* codes, const uint8_t* const* sel,
                              const float* const* tin, float* const* tout, int flags,
                              const double* err, const double* w2, const char* who) {
  aaac_status st = check_batch(count, W, R, C, g, S, n, who);
  if (st != AAAC_OK) return st;
  if (flags & ~(AAAC_REFINE_ROUND_BF16 | AAAC_REFINE_W2_KNOWN))
    return fail(AAAC_ERR_INVALID_ARG, "%s: unknown flags %d", who, flags);
  if (!I || !codes || !sel || !tin || !tout) return fail(AAAC_ERR_INVALID_ARG, "%s: null array", who);
  for (int i = 0; i < count; ++i) {
    if (!I[i] || !aligned(I[i], 16) || !codes[i] || !aligned(codes[i], 16) || !sel[i] || !tin[i] ||
        !tout[i] || !aligned(tin[i], 4) || !aligned(tout[i], 4))
      return fail(AAAC_ERR_INVALID_ARG, "%s: matrix %d: null or misaligned pointer", who, i);
  }
  if (err && (!aligned(err, 8) || !w2 || !aligned(w2, 8)))
    return fail(AAAC_ERR_INVALID_ARG, "%s: err and w2 must be given together, 8-byte aligned", who);
  if (!err && (flags & AAAC_REFINE_W2_KNOWN))
    return fail(AAAC_ERR_INVALID_ARG, "%s: AAAC_REFINE_W2_KNOWN without err and w2", who);
  return AAAC_OK;
}

aaac_status do_refine(int count, const uint16_t* const* W, const int64_t* R, const int64_t* C,
                      int g, int S, int n, const float* const* I, const uint8_t* const* codes,
                      const uint8_t* const* sel, const float* const* tin, float* const* tout,
                      int flags, double* err, double* w2, void* ws, size_t ws_bytes, void* stream,
                      const char* who, bool clear_counters = false) {
  aaac_status st = check_refine_args(count, W, R, C, g, S, n, I, codes, sel, tin, tout, flags, err,
                                     w2, who);
  if (st != AAAC_OK) return st;
  st = check_refine_ws(count, ws, ws_bytes, who);
  if (st != AAAC_OK) return st;
  if (clear_counters) {
    // every argument is valid: clear the job counters first (a call that did not complete may
    // have left them set)
    hipLaunchKernelGGL(clear_words_kernel, dim3(1), dim3(64), 0,
                       static_cast<hipStream_t>(stream), static_cast<uint32_t*>(ws), 64);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_status(e, who);
  }
  RefineBatch b{};
  build_refine_batch(b, count, W, R, C, g, S, n, I, flags, ws);
  b.errs = err ? 1 : 0;
  for (int i = 0; i < count; ++i) {
    RefineJob& j = b.job[i];
    j.codes = reinterpret_cast<const uint32_t*>(codes[i]);
    j.sel = sel[i];
    j.tables_in = tin[i];
    j.tables_out = tout[i];
    j.err_out = err ? err + i : nullptr;
    j.err_after = err ? err + count + i : nullptr;
    j.w2 = err ? w2 + i : nullptr;
  }
  return hip_status(launch_refine(b, static_cast<hipStream_t>(stream)), who);
}


aaac_status do_gemv(int count, const uint8_t* const* codes, const uint16_t* const* scales,
                    const uint8_t* const* bitmap, const uint16_t* const* tables,
                    const int64_t* R, const int64_t* C, int g, int S, int n,
                    const uint16_t* const* x, int B, float* const* y, void* stream,
                    const char* who) {
  if (count < 1 || count > AAAC_MAX_BATCH || !codes || !scales || !tables || !R || !C || !x || !y)
    return fail(AAAC_ERR_INVALID_ARG, "%s: count=%d (need 1..%d) and non-null arrays", who, count,
                AAAC_MAX_BATCH);
  if (B < 1 || B > 4) return fail(AAAC_ERR_UNSUPPORTED_SHAPE, "%s: B=%d (need 1..4)", who, B);
  int order[AAAC_MAX_BATCH];
  for (int i = 0; i < count; ++i) {
    aaac_status st = check_shape(R[i], C[i], g, S, n, true, who);
    if (st != AAAC_OK) return st;
    if (C[i] % 32 != 0)
      return fail(AAAC_ERR_UNSUPPORTED_SHAPE, "%s: C=%lld (need C %% 32 == 0)", who,
                  (long long)C[i]);
    const uint8_t* bm = bitmap ? bitmap[i] : nullptr;
    if (!codes[i] || !aligned(codes[i], 16) || !scales[i] || !aligned(scales[i], 8) ||
        !tables[i] || !aligned(tables[i], 2) || !x[i] || !aligned(x[i], 16) || !y[i] ||
        !aligned(y[i], 4))
      return fail(AAAC_ERR_INVALID_ARG, "%s: matrix %d: null or misaligned pointer", who, i);
    if ((S < g) != (bm != nullptr))
      return fail(AAAC_ERR_INVALID_ARG, "%s: bitmap must be given exactly when S < g", who);
    // widest matrices first: their tasks are the longest, so they start first
    int k = i;
    while (k > 0 && C[order[k - 1]] < C[i]) {
      order[k] = order[k - 1];
      --k;
    }
    order[k] = i;
  }
  GemvBatch b = {};
  b.njobs = count;
  b.B = B;
  b.g = g;
  b.S = S;
  b.n = n;
  int64_t t = 0;
  for (int k = 0; k < count; ++k) {
    const int i = order[k];
    GemvJob& jb = b.job[k];
    jb.codes = codes[i];
    jb.scales = scales[i];
    jb.bitmap = bitmap ? bitmap[i] : nullptr;
    jb.tables = tables[i];
    jb.x = x[i];
    jb.y = y[i];
    jb.R = R[i];
    jb.C = C[i];
    jb.task_begin = t;
    jb.split = gemv_split(C[i]);
    t += gemv_tasks(R[i], C[i]);
  }
  b.total_tasks = t;
  return hip_status(launch_gemv(b, static_cast<hipStream_t>(stream)), who);
}

aaac_status do_init(int count, const uint16_t* const* W, const int64_t* R, const int64_t* C,
                    int g, int n, float* const* tables, void* ws, size_t ws_bytes, void* stream,
                    const char* who) {
  if (count < 1 || count > AAAC_MAX_BATCH)
    return fail(AAAC_ERR_INVALID_ARG, "%s: count=%d (need 1..%d)", who, count, AAAC_MAX_BATCH);
  if (!W || !R || !C || !tables) return fail(AAAC_ERR_INVALID_ARG, "%s: null array", who);
  for (int i = 0; i < count; ++i) {
    aaac_status st = check_shape(R[i], C[i], g, 8, n, false, who);
    if (st != AAAC_OK) return st;
    if (!W[i] || !aligned(W[i], 16) || !tables[i] || !aligned(tables[i], 4))
      return fail(AAAC_ERR_INVALID_ARG, "%s: matrix %d: W or tables null or misaligned", who, i);
  }
  const size_t need = init_workspace_bytes(count, R, C);
  if (!ws || !aligned(ws, 256)) return fail(AAAC_ERR_INVALID_ARG, "%s: ws null or not 256-byte aligned", who);
  if (ws_bytes < need)
    return fail(AAAC_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu < %zu bytes", who, ws_bytes, need);
  return hip_status(launch_init(count, W, R, C, g, n, tables, ws, static_cast<hipStream_t>(stream)),
                    who);
}


aaac_status do_pack(int count, const uint16_t* const* W, const int64_t* R, const int64_t* C, int g,
                    int S, int n, const uint8_t* const* sel, const float* const* tables,
                    uint16_t* const* scales, uint8_t* const* bitmap, uint16_t* const* tables_bf16,
                    void* stream, const char* who) {
  if (count < 1 || count > AAAC_MAX_BATCH)
    return fail(AAAC_ERR_INVALID_ARG, "%s: count %d outside [1, %d]", who, count, AAAC_MAX_BATCH);
  if (!W || !R || !C || !sel || !tables || !scales || !tables_bf16)
    return fail(AAAC_ERR_INVALID_ARG, "%s: null array", who);
  for (int i = 0; i < count; ++i) {
    aaac_status st = check_shape(R[i], C[i], g, S, n, true, who);
    if (st != AAAC_OK) return st;
    if (!W[i] || !aligned(W[i], 16) || !sel[i] || !tables[i] || !aligned(tables[i], 4) ||
        !scales[i] || !aligned(scales[i], 2) || !tables_bf16[i] || !aligned(tables_bf16[i], 2))
      return fail(AAAC_ERR_INVALID_ARG, "%s: null or misaligned pointer (matrix %d)", who, i);
    const uint8_t* bm = bitmap ? bitmap[i] : nullptr;
    if ((S < g) != (bm != nullptr))
      return fail(AAAC_ERR_INVALID_ARG, "%s: bitmap must be given exactly when S < g", who);
  }
  return hip_status(launch_pack(count, W, R, C, g, S, n, sel, tables, scales, bitmap, tables_bf16,
                                static_cast<hipStream_t>(stream)),
                    who);
}

aaac_status do_dequant(int count, const uint8_t* const* codes, const uint16_t* const* scales,
                       const uint8_t* const* bitmap, const uint16_t* const* tables_bf16,
                       const int64_t* R, const int64_t* C, int g, int S, int n,
                       uint16_t* const* W_hat, void* stream, const char* who) {
  if (count < 1 || count > AAAC_MAX_BATCH)
    return fail(AAAC_ERR_INVALID_ARG, "%s: count %d outside [1, %d]", who, count, AAAC_MAX_BATCH);
  if (!codes || !scales || !tables_bf16 || !R || !C || !W_hat)
    return fail(AAAC_ERR_INVALID_ARG, "%s: null array", who);
  for (int i = 0; i < count; ++i) {
    aaac_status st = check_shape(R[i], C[i], g, S, n, true, who);
    if (st != AAAC_OK) return st;
    if (!codes[i] || !aligned(codes[i], 4) || !scales[i] || !aligned(scales[i], 2) ||
        !tables_bf16[i] || !aligned(tables_bf16[i], 2) || !W_hat[i] || !aligned(W_hat[i], 16))
      return fail(AAAC_ERR_INVALID_ARG, "%s: null or misaligned pointer (matrix %d)", who, i);
    const uint8_t* bm = bitmap ? bitmap[i] : nullptr;
    if ((S < g) != (bm != nullptr))
      return fail(AAAC_ERR_INVALID_ARG, "%s: bitmap must be given exactly when S < g", who);
  }
  return hip_status(launch_dequant(count, codes, scales, bitmap, tables_bf16, R, C, g, S, n,
                                   W_hat, static_cast<hipStream_t>(stream)),
                    who);
}

}  // namespace

extern "C" {

const char* aaac_status_string(aaac_status status) {
  switch (status) {
    case AAAC_OK: return "ok";
    case AAAC_ERR_INVALID_ARG: return "invalid argument";
    case AAAC_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
    case AAAC_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case AAAC_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* aaac_last_error(void) { return g_err; }

size_t aaac_workspace_bytes(int op, int64_t R, int64_t C, int g, int S, int n) {
  switch (op) {
    case AAAC_OP_IMPORTANCE: {
      if (R < 0 || C < 1) return 0;
      const int ns = importance_splits(R, C);
      return ns > 0 ? (size_t)ns * (size_t)C * sizeof(double) : 256;
    }
    case AAAC_OP_INIT:
      if (check_shape(R, C, g, 8, n, false, "aaac_workspace_bytes") != AAAC_OK) return 0;
      return init_workspace_bytes(1, &R, &C);
    case AAAC_OP_ASSIGN:
      if (check_shape(R, C, g, S, n, true, "aaac_workspace_bytes") != AAAC_OK) return 0;
      return assign_ws_bytes(1);
    case AAAC_OP_REFINE:
      if (check_shape(R, C, g, S, n, true, "aaac_workspace_bytes") != AAAC_OK) return 0;
      return refine_ws_bytes(1);
    default:
      return 0;
  }
}

size_t aaac_batch_workspace_bytes(int op, int count, const int64_t* R, const int64_t* C, int g,
                                  int S, int n) {
  if (count < 1 || count > AAAC_MAX_BATCH || !R || !C) return 0;
  const bool init = op == AAAC_OP_INIT;
  for (int i = 0; i < count; ++i)
    if (check_shape(R[i], C[i], g, init ? 8 : S, n, !init, "aaac_batch_workspace_bytes") != AAAC_OK)
      return 0;
  if (op == AAAC_OP_REFINE) return refine_ws_bytes(count);
  if (op == AAAC_OP_ASSIGN) return assign_ws_bytes(count);
  if (init) return init_workspace_bytes(count, R, C);
  return 0;
}

aaac_status aaac_importance(const float* X, int64_t T, int64_t K, int64_t ldx, double* I_acc,
                            float* I_out, void* ws, size_t ws_bytes, void* stream) {
  const char* who = "aaac_importance";
  if (T < 0 || K < 1 || ldx < K)
    return fail(AAAC_ERR_UNSUPPORTED_SHAPE, "%s: T=%lld K=%lld ldx=%lld", who, (long long)T,
                (long long)K, (long long)ldx);
  if ((T > 0 && !X) || !I_acc || !aligned(I_acc, 8) || (I_out && !aligned(I_out, 4)) ||
      (X && !aligned(X, 4)))
    return fail(AAAC_ERR_INVALID_ARG, "%s: null or misaligned pointer", who);
  const int ns = importance_splits(T, K);
  const size_t need = ns > 0 ? (size_t)ns * (size_t)K * sizeof(double) : 0;
  if (need && (!ws || !aligned(ws, 256)))
    return fail(AAAC_ERR_INVALID_ARG, "%s: ws null or not 256-byte aligned", who);
  if (ws_bytes < need)
    return fail(AAAC_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu < %zu bytes", who, ws_bytes, need);
  return hip_status(launch_importance(X, T, K, ldx, I_acc, I_out, static_cast<double*>(ws), ns,
                                      static_cast<hipStream_t>(stream)),
                    who);
}

aaac_status aaac_init_quantiles(const uint16_t* W, int64_t R, int64_t C, int g, int n,
                                float* tables, void* ws, size_t ws_bytes, void* stream) {
  return do_init(1, &W, &R, &C, g, n, &tables, ws, ws_bytes, stream, "aaac_init_quantiles");
}

aaac_status aaac_init_quantiles_batch(int count, const uint16_t* const* W, const int64_t* R,
                                      const int64_t* C, int g, int n, float* const* tables,
                                      void* ws, size_t ws_bytes, void* stream) {
  return do_init(count, W, R, C, g, n, tables, ws, ws_bytes, stream, "aaac_init_quantiles_batch");
}

aaac_status aaac_assign(const uint16_t* W, int64_t R, int64_t C, int g, int S, int n,
                        const float* I, const float* tables, uint8_t* codes, uint8_t* sel,
                        double* err, double* err_total, void* ws, size_t ws_bytes, void* stream) {
  return do_assign(1, &W, &R, &C, g, S, n, &I, &tables, &codes, &sel, err, err_total, ws, ws_bytes,
                   stream, "aaac_assign");
}

aaac_status aaac_assign_batch(int count, const uint16_t* const* W, const int64_t* R,
                              const int64_t* C, int g, int S, int n, const float* const* I,
                              const float* const* tables, uint8_t* const* codes,
                              uint8_t* const* sel, double* err_total, void* ws, size_t ws_bytes,
                              void* stream) {
  return do_assign(count, W, R, C, g, S, n, I, tables, codes, sel, nullptr, err_total, ws,
                   ws_bytes, stream, "aaac_assign_batch");
}

aaac_status aaac_refine(const uint16_t* W, int64_t R, int64_t C, int g, int S, int n,
                        const float* I, const uint8_t* codes, const uint8_t* sel,
                        const float* tables_in, float* tables_out, int flags, double* err,
                        double* w2, void* ws, size_t ws_bytes, void* stream) {
  return do_refine(1, &W, &R, &C, g, S, n, &I, &codes, &sel, &tables_in, &tables_out, flags, err,
                   w2, ws, ws_bytes, stream, "aaac_refine");
}

aaac_status aaac_refine_batch(int count, const uint16_t* const* W, const int64_t* R,
                              const int64_t* C, int g, int S, int n, const float* const* I,
                              const uint8_t* const* codes, const uint8_t* const* sel,
                              float* const* tables, int flags, double* err, double* w2, void* ws,
                              size_t ws_bytes, void* stream) {
  if (!tables) return fail(AAAC_ERR_INVALID_ARG, "aaac_refine_batch: null tables array");
  const float* tin[AAAC_MAX_BATCH];
  const int m = count < AAAC_MAX_BATCH ? (count > 0 ? count : 0) : AAAC_MAX_BATCH;
  for (int i = 0; i < m; ++i) tin[i] = tables[i];
  return do_refine(count, W, R, C, g, S, n, I, codes, sel, tin, tables, flags, err, w2, ws,
                   ws_bytes, stream, "aaac_refine_batch");
}

aaac_status aaac_refine_batch_noalloc(int count, const uint16_t* const* W, const int64_t* R,
                                      const int64_t* C, int g, int S, int n,
                                      const float* const* I, const uint8_t* const* codes,
                                      const uint8_t* const* sel, float* const* tables, int flags,
                                      double* err, double* w2, void* stream) {
  const char* who = "aaac_refine_batch_noalloc";
  if (!tables) return fail(AAAC_ERR_INVALID_ARG, "%s: null tables array", who);
  if (count < 1 || count > AAAC_MAX_BATCH)
    return fail(AAAC_ERR_INVALID_ARG, "%s: count=%d (need 1..%d)", who, count, AAAC_MAX_BATCH);
  const size_t need = refine_ws_bytes(count);
  if (need > kScratchBytes)
    return fail(AAAC_ERR_WORKSPACE_TOO_SMALL, "%s: needs %zu bytes of scratch, the fixed maximum is "
                "%zu", who, need, kScratchBytes);
  const float* tin[AAAC_MAX_BATCH];
  for (int i = 0; i < count; ++i) tin[i] = tables[i];
  // every argument first, then the scratch address (the first call on a device looks it up)
  aaac_status st = check_refine_args(count, W, R, C, g, S, n, I, codes, sel, tin, tables, flags,
                                     err, w2, who);
  if (st != AAAC_OK) return st;
  void* ws = scratch_on_current_device(who, &st);
  if (!ws) return st;
  return do_refine(count, W, R, C, g, S, n, I, codes, sel, tin, tables, flags, err, w2, ws,
                   kScratchBytes, stream, who, /*clear_counters=*/true);
}

aaac_status aaac_pack(const uint16_t* W, int64_t R, int64_t C, int g, int S, int n,
                      const uint8_t* sel, const float* tables, const uint8_t* codes_u8,
                      uint8_t* codes_out, uint16_t* scales, uint8_t* bitmap,
                      uint16_t* tables_bf16, void* stream) {
  const char* who = "aaac_pack";
  if ((codes_u8 != nullptr) != (codes_out != nullptr))
    return fail(AAAC_ERR_INVALID_ARG, "%s: codes_u8 and codes_out must be given together", who);
  if (codes_u8 && (!aligned(codes_u8, 8) || !aligned(codes_out, 4)))
    return fail(AAAC_ERR_INVALID_ARG, "%s: codes_u8 needs 8-byte and codes_out 4-byte alignment",
                who);
  uint8_t* const bm[1] = {bitmap};
  aaac_status st = do_pack(1, &W, &R, &C, g, S, n, &sel, &tables, &scales, bm, &tables_bf16,
                           stream, who);
  if (st != AAAC_OK || !codes_u8) return st;
  return hip_status(launch_pack_codes(codes_u8, codes_out, R, C, static_cast<hipStream_t>(stream)),
                    who);
}

aaac_status aaac_pack_batch(int count, const uint16_t* const* W, const int64_t* R,
                            const int64_t* C, int g, int S, int n, const uint8_t* const* sel,
                            const float* const* tables, uint16_t* const* scales,
                            uint8_t* const* bitmap, uint16_t* const* tables_bf16, void* stream) {
  return do_pack(count, W, R, C, g, S, n, sel, tables, scales, bitmap, tables_bf16, stream,
                 "aaac_pack_batch");
}

aaac_status aaac_dequant(const uint8_t* codes, const uint16_t* scales, const uint8_t* bitmap,
                         const uint16_t* tables_bf16, int64_t R, int64_t C, int g, int S, int n,
                         uint16_t* W_hat, void* stream) {
  const uint8_t* const bm[1] = {bitmap};
  return do_dequant(1, &codes, &scales, bm, &tables_bf16, &R, &C, g, S, n, &W_hat, stream,
                    "aaac_dequant");
}

aaac_status aaac_dequant_batch(int count, const uint8_t* const* codes,
                               const uint16_t* const* scales, const uint8_t* const* bitmap,
                               const uint16_t* const* tables_bf16, const int64_t* R,
                               const int64_t* C, int g, int S, int n, uint16_t* const* W_hat,
                               void* stream) {
  return do_dequant(count, codes, scales, bitmap, tables_bf16, R, C, g, S, n, W_hat, stream,
                    "aaac_dequant_batch");
}

aaac_status aaac_assign_refine_batch(int count, const uint16_t* const* W, const int64_t* R,
                                     const int64_t* C, int g, int S, int n,
                                     const float* const* I, float* const* tables,
                                     uint8_t* const* codes, uint8_t* const* sel, int flags,
                                     double* err, double* w2, void* ws, size_t ws_bytes,
                                     void* stream) {
  const char* who = "aaac_assign_refine_batch";
  if (count < 1 || count > AAAC_MAX_BATCH || !tables || !codes || !sel)
    return fail(AAAC_ERR_INVALID_ARG, "%s: count=%d (need 1..%d) and non-null arrays", who, count,
                AAAC_MAX_BATCH);
  const float* tin[AAAC_MAX_BATCH];
  const uint8_t* cc[AAAC_MAX_BATCH];
  const uint8_t* sc[AAAC_MAX_BATCH];
  for (int i = 0; i < count; ++i) {
    tin[i] = tables[i];
    cc[i] = codes[i];
    sc[i] = sel[i];
  }
  aaac_status st = check_refine_args(count, W, R, C, g, S, n, I, cc, sc, tin, tables, flags, err,
                                     w2, who);
  if (st != AAAC_OK) return st;
  st = check_refine_ws(count, ws, ws_bytes, who);
  if (st != AAAC_OK) return st;
  if (S < kWideLane) {
    // 8-weight selection groups: the two launches
    st = do_assign(count, W, R, C, g, S, n, I, tin, codes, sel, nullptr, nullptr, nullptr, 0,
                   stream, who);
    if (st != AAAC_OK) return st;
    return do_refine(count, W, R, C, g, S, n, I, cc, sc, tin, tables, flags, err, w2, ws,
                     ws_bytes, stream, who);
  }
  RefineBatch b{};
  build_refine_batch(b, count, W, R, C, g, S, n, I, flags, ws);
  b.errs = err ? 1 : 0;
  for (int i = 0; i < count; ++i) {
    RefineJob& j = b.job[i];
    j.codes = reinterpret_cast<const uint32_t*>(codes[i]);
    j.sel = sel[i];
    j.codes_out = reinterpret_cast<uint32_t*>(codes[i]);
    j.sel_out = sel[i];
    j.tables_in = tables[i];
    j.tables_out = tables[i];
    j.err_out = err ? err + i : nullptr;
    j.err_after = err ? err + count + i : nullptr;
    j.w2 = err ? w2 + i : nullptr;
  }
  return hip_status(launch_assign_refine(b, static_cast<hipStream_t>(stream)), who);
}

aaac_status aaac_awq_prescale(const uint16_t* W, int64_t R, int64_t C, const float* a,
                              const float* I, uint16_t* W_scaled, float* I_scaled, void* stream) {
  const char* who = "aaac_awq_prescale";
  if (R < 1 || C < 8 || C % 8 != 0 || C >= ((int64_t)1 << 31) ||
      R > ((((int64_t)1 << 40) - 1) / C))
    return fail(AAAC_ERR_UNSUPPORTED_SHAPE,
                "%s: R=%lld C=%lld (need R >= 1, C >= 8, C %% 8 == 0, R*C < 2^40)", who,
                (long long)R, (long long)C);
  if (!W || !aligned(W, 16) || !a || !aligned(a, 16) || !W_scaled || !aligned(W_scaled, 16))
    return fail(AAAC_ERR_INVALID_ARG, "%s: null or misaligned pointer", who);
  if ((I == nullptr) != (I_scaled == nullptr) || (I && (!aligned(I, 4) || !aligned(I_scaled, 4))))
    return fail(AAAC_ERR_INVALID_ARG, "%s: I and I_scaled must be given together, 4-byte aligned",
                who);
  return hip_status(launch_awq_prescale(W, R, C, a, I, W_scaled, I_scaled,
                                        static_cast<hipStream_t>(stream)),
                    who);
}

aaac_status aaac_gemv(const uint8_t* codes, const uint16_t* scales, const uint8_t* bitmap,
                      const uint16_t* tables_bf16, int64_t R, int64_t C, int g, int S, int n,
                      const uint16_t* x, int B, float* y, void* stream) {
  return do_gemv(1, &codes, &scales, bitmap ? &bitmap : nullptr, &tables_bf16, &R, &C, g, S, n,
                 &x, B, &y, stream, "aaac_gemv");
}

aaac_status aaac_gemv_batch(int count, const uint8_t* const* codes, const uint16_t* const* scales,
                            const uint8_t* const* bitmap, const uint16_t* const* tables_bf16,
                            const int64_t* R, const int64_t* C, int g, int S, int n,
                            const uint16_t* const* x, int B, float* const* y, void* stream) {
  return do_gemv(count, codes, scales, bitmap, tables_bf16, R, C, g, S, n, x, B, y, stream,
                 "aaac_gemv_batch");
}

}  // extern "C"
