// Host side of libfd: argument checks, workspace layout, split planner and
// kernel dispatch behind the C ABI declared in include/fd.h.
//
// Argument rules mirror the host checks of flash_decode_splitk in
// "flash_decode_splitk.py" (MiniInfer) -- supported head dims, positive
// sizes, heads a multiple of kv_heads, positive split count -- returned as
// status codes instead of exceptions. The planner follows the split-count
// guidance of "04_flash_decoding.py" (CS349E lecture 11), demo 4, the
// 256-keys-per-split default of flash_decode_splitk.py, and the rule of
// "decode_attention_splitkv.py" (TileLang tutorial, ch. 18) that no split may
// be empty.
#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/fd.h"
#include "fd_internal.h"
#include "fd_steal.h"

// Partials of fd_decode_attention_noalloc: one array per GPU, resident from
// module load until the process ends. In host code `scratch` names a host-side
// stand-in, not device memory: its device address on the current GPU comes
// from hipGetSymbolAddress (scratch_on_device below) and only that address
// is ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[FD_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_last_error[256] = "";
// Split-kernel choice of fd_set_kernel_path: per thread, so callers on
// different threads never steer each other's launches.
thread_local int g_path = FD_PATH_AUTO;
// Schedule of the split launch (fd_set_schedule) and where whole calls
// merge the partials (fd_set_combine), per thread like the path.
thread_local int g_sched = FD_SCHED_AUTO;
thread_local int g_combine = FD_COMBINE_SEPARATE;

// The library's own choice of split kernel: matrix-core QK^T wherever that
// kernel exists (head dim 128) and the group has at least 2 query heads.
// Measured on MI355X: with 16-bit inputs and both kernels streaming whole
// K/V rows, the matrix-core kernel is 0-15 % faster at groups 2-8 (2.5-2.8x
// fewer VALU instructions at 4-8), while at group 1 -- one valid column of
// its 16 -- the VALU kernel is 1-5 % faster. With fp32 inputs
// (v_mfma_f32_16x16x4_f32) it is level where the launch is bandwidth-bound
// (B16 x 4096 keys, 32/8 heads: 85.3 vs 84.4 us) and faster where the VALU
// kernel's 32-lane dot-product reductions bound it: the 8:1 exactness case
// (one sequence of 10,000 keys, 7 splits) 68.7 -> 37.6 us, B4 x 16384 keys
// 68.2 -> 49.6 us, B64 x 1024 keys 37.1 -> 28.7 us per call.
bool auto_mfma(int dtype, int dim, int group) {
  (void)dtype;
  return dim == 128 && group >= 2;
}

int hip_fail(hipError_t e, const char* where) {
  std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%d)", where, hipGetErrorString(e),
                (int)e);
  return FD_ERR_HIP;
}

constexpr double kLog2e = 1.4426950408889634074;
constexpr int64_t kMaxWorkgroups = int64_t(1) << 24;
// Fewest keys per split the planner will create (flash_decode_splitk.py's
// default of one split per 256 keys).
constexpr int kPlanMinKeysPerSplit = 256;
// Time model of one call (split launch + combine launch), fitted on MI355X
// to 74 measured calls -- the split-count sweeps of 04_flash_decoding.py
// demo 4 (16/2 heads at B1 x 64K, B8 x 8K, B64 x 2K, 14 split counts each)
// and four Llama-8B-shaped sweeps -- with relative RMS error 4.7 % (largest
// 15 %); `python bench.py --fit-planner` re-measures and refits. A launch of
// w workgroups runs rounds of min(CUs, remaining) workgroups; a round costs
// a fixed workgroup time plus its bytes at a per-byte time that grows with
// the number of workgroups streaming at once (one workgroup alone streams
// ~51 GB/s; 256 together ~27 GB/s each):
//   T_split = launch + sum over rounds (workgroup + bytes * (1/rate + n/contention))
//   T_call  = T_split + [ns > 1] (combine + combine_per_mb * partial MB)
constexpr double kModelLaunchUs = 3.848;
constexpr double kModelWorkgroupUs = 0.972;
constexpr double kModelRateBytesPerUs = 50960.0;          // one workgroup alone
constexpr double kModelContentionBytesPerUs = 14.825e6;   // n/this: per-byte time of n at once
constexpr double kModelCombineUs = 2.537;
constexpr double kModelCombineUsPerMB = 0.7034;           // per MB of fp32 partials

// Compute units of the current device, cached per device ordinal.
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

int device_cus(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev >= 0 && dev < kMaxDevices) {
    const int c = g_cus[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *cus = c;
      return FD_OK;
    }
  }
  int c = 0;
  e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
  if (dev >= 0 && dev < kMaxDevices) g_cus[dev].store(c, std::memory_order_relaxed);
  *cus = c;
  return FD_OK;
}

// Device address of `scratch` on the current GPU, looked up once per device
// (with that device current) and cached.
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_on_device(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) {
    std::snprintf(g_last_error, sizeof(g_last_error), "device ordinal %d beyond %d", dev,
                  kMaxDevices);
    return FD_ERR_UNSUPPORTED;
  }
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
      if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 255u) != 0) {
        std::snprintf(g_last_error, sizeof(g_last_error), "scratch address %p not 256-B aligned",
                      p);
        return FD_ERR_HIP;
      }
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return FD_OK;
}

int elem_bytes(int dtype) { return dtype == FD_F32 ? 4 : 2; }

bool dim_ok(int dim) { return dim == 16 || dim == 32 || dim == 64 || dim == 128; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Sizes {
  int group, rows, row_chunks;
  int64_t workgroups;
};

// Query rows of a GQA group one workgroup handles: up to 8 (the packed
// group), or 1 for the unpacked comparison path.
int rows_per_pass(int path) { return path == FD_PATH_UNPACKED ? 1 : fd::kMaxRowsPerPass; }

// Checks shared by every launching entry point.
int check_common(int batch, int heads, int kv_heads, int dim, int num_splits, int dtype,
                 Sizes* sz, int max_rows = fd::kMaxRowsPerPass) {
  if (batch < 1 || heads < 1 || kv_heads < 1 || num_splits < 1) return FD_ERR_INVALID_ARG;
  if (heads % kv_heads != 0) return FD_ERR_INVALID_ARG;
  if (num_splits > FD_MAX_SPLITS) return FD_ERR_INVALID_ARG;
  if (dtype != FD_F32 && dtype != FD_F16 && dtype != FD_BF16) return FD_ERR_UNSUPPORTED;
  if (!dim_ok(dim)) return FD_ERR_UNSUPPORTED;
  const int group = heads / kv_heads;
  if (group > FD_MAX_GROUP) return FD_ERR_UNSUPPORTED;
  sz->group = group;
  sz->rows = group < max_rows ? group : max_rows;
  sz->row_chunks = (group + max_rows - 1) / max_rows;
  sz->workgroups = (int64_t)batch * kv_heads * sz->row_chunks * num_splits;
  if (sz->workgroups > kMaxWorkgroups) return FD_ERR_INVALID_ARG;
  if ((int64_t)batch * heads > INT_MAX / 2) return FD_ERR_INVALID_ARG;
  return FD_OK;
}

int check_layout(const fd_kv_layout* lay, int kv_heads, int dim, int dtype, fd_kv_layout* out) {
  fd_kv_layout L;
  if (lay == nullptr) {
    L.batch_stride = 0;
    L.head_stride = dim;
    L.token_stride = (int64_t)kv_heads * dim;
    L.cu_stride = (int64_t)kv_heads * dim;
  } else {
    L = *lay;
  }
  if (L.batch_stride < 0 || L.head_stride < 0 || L.token_stride < dim || L.cu_stride < 0)
    return FD_ERR_INVALID_ARG;
  const int64_t eb = elem_bytes(dtype);
  const int64_t s[4] = {L.batch_stride, L.head_stride, L.token_stride, L.cu_stride};
  for (int64_t x : s)
    if ((x * eb) % 16 != 0) return FD_ERR_INVALID_ARG;
  // Offsets inside one tile are 32-bit: keep a tile (<= 128 keys) far
  // below 2^32 bytes.
  if (L.token_stride * eb > (int64_t(1) << 23)) return FD_ERR_INVALID_ARG;
  *out = L;
  return FD_OK;
}

// The two workspace formats.
//   kNormalised: Opart [B,H,ns,D] o_s, then (256-B aligned) LSE [B,ns,H]
//                (decode_attention_splitkv.py's part_shape / lse_shape),
//                then (256-B aligned) the control block: the claim counter
//                of a queue-scheduled launch (first int32 of 256 bytes),
//                then int32 arrival counters [B*H] of fused calls (256-B
//                aligned size), which must be zero before a fused call and
//                are left zero by it.
//   kUnnorm:     ACC [B,H,ns,D] acc_s, then (256-B aligned) M [B,H,ns],
//                then (256-B aligned) L [B,H,ns] (flash_decode_splitk.py's
//                ACC_BUF, M_BUF, L_BUF), with ceil-equal split bounds.
enum Format { kNormalised = 0, kUnnorm = 1 };

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Workspace {
  float* opart = nullptr;
  float* lse = nullptr;
  float* mbuf = nullptr;
  float* lbuf = nullptr;
  int* queue = nullptr;     // claim counter (normalised format)
  int* arrivals = nullptr;  // arrival counters of fused calls (normalised format)
  unsigned long long* steal = nullptr;  // share words of the steal schedule (normalised format)
};

constexpr size_t kQueueBytes = 256;
constexpr size_t kStealBytes = (size_t)fd::kStealMaxShares * sizeof(unsigned long long);

size_t control_bytes(int batch, int heads) {
  return kQueueBytes + align256((size_t)batch * heads * sizeof(int)) + kStealBytes;
}

size_t workspace_bytes(Format f, int batch, int heads, int dim, int num_splits) {
  const size_t rows = (size_t)batch * heads * num_splits;
  const size_t opart = align256(rows * dim * sizeof(float));
  if (f == kNormalised)
    return opart + align256(rows * sizeof(float)) + control_bytes(batch, heads);
  return opart + align256(rows * sizeof(float)) + rows * sizeof(float);
}

Workspace workspace_views(Format f, void* base, int batch, int heads, int dim, int num_splits) {
  char* ws = static_cast<char*>(base);
  const size_t rows = (size_t)batch * heads * num_splits;
  const size_t opart = align256(rows * dim * sizeof(float));
  Workspace w;
  w.opart = reinterpret_cast<float*>(ws);
  if (f == kNormalised) {
    w.lse = reinterpret_cast<float*>(ws + opart);
    w.queue = reinterpret_cast<int*>(ws + opart + align256(rows * sizeof(float)));
    w.arrivals = reinterpret_cast<int*>(ws + opart + align256(rows * sizeof(float)) + kQueueBytes);
    w.steal = reinterpret_cast<unsigned long long*>(
        ws + opart + align256(rows * sizeof(float)) + kQueueBytes +
        align256((size_t)batch * heads * sizeof(int)));
  } else {
    w.mbuf = reinterpret_cast<float*>(ws + opart);
    w.lbuf = reinterpret_cast<float*>(ws + opart + align256(rows * sizeof(float)));
  }
  return w;
}

// FD_SCHED_AUTO keeps the static schedule. Measured on MI355X (same split
// count, A/B in one process), the queue schedule with one workgroup per
// compute unit wins only on ragged batches: varlen Qwen (32 sequences of
// 64..32768 keys, 8 splits) 201.9 -> 187.2 us; it loses on uniform lengths,
// where each extra segment a workgroup walks exposes its fixed costs
// (Llama B16/8K +2.5 % at 8 splits, +9 % at 16; flash-decoding B64/2K
// +24 %, B8/8K at 64 splits +32 %; MHA +19..49 %). The lengths are on the
// device, so the host cannot tell the cases apart: callers with ragged
// batches select FD_SCHED_QUEUE.
bool use_queue(int sched) { return sched == FD_SCHED_QUEUE; }

// Target chunks per share of the steal schedule (each chunk at least
// fd::kStealMinChunk keys, so shorter shares have fewer). Measured on
// MI355X, Llama B16/128K (bf16, 8 slots: 2 shares per unit, 3 steal slots
// each), whole call in graph replay, static schedule at the planner's 2
// splits 1295-1330 us on that device: 1 chunk (no claims) 1281-1285 us,
// 4: 1281, 16: 1262-1269, 32: 1239-1240, 64: 1237-1239.
#ifndef FD_STEAL_CHUNKS
#define FD_STEAL_CHUNKS 32
#endif
constexpr int kStealChunks = FD_STEAL_CHUNKS;
static_assert(kStealChunks >= 1 && kStealChunks <= fd::kStealMaxChunks,
              "the share word's front and back counts hold at most kStealMaxChunks");
// Steal slots per share in the planner's layout for the steal schedule.
constexpr int kStealPlanCap = 3;
// fd_plan_schedule's rule for the steal schedule. Measured on MI355X, whole
// calls in graph replay against the static schedule at the planner's split
// count, Llama-3.1-8B shapes (bf16, 32/8 heads): every share streaming
// 16.8-67 MB with lengths within 2x gains 1-8 % (B16 x 64K, 128K, 256K;
// B8 x 256K; B4 x 512K; B2 x 1M; B16 x 64K-128K ragged), B32 x 64K (one
// share per unit) is level, lengths within 3.7x gain 0.9 %; shares of
// 8.4 MB (B16 x 32K) lose 1-3 %, of 2 MB (B1 x 128K) 7 %, and ragged
// Qwen-shaped batches of 1-1.6 GB lose 0-10 %.
constexpr int64_t kStealPlanMaxRatio = 4;
constexpr double kStealPlanMinShareBytes = 12e6;
// fd_plan_schedule's rule for ragged batches (longest >= 1.5x shortest):
// the queue schedule with about this many segments per compute unit.
// Measured on MI355X, whole calls in graph replay: on every ragged batch
// tried (Qwen-shaped B32 with lengths 1K-32K, 8K-32K, 16K-32K and 64-32K;
// Llama-shaped B16 with 32K-128K and 64K-128K; B4 with 8K-64K) the queue at
// 4 segments per CU was the fastest option or within 1.3 % of it (e.g.
// Qwen 1K-32K: 161 us against 169-180 static at 12-28 splits and 168-188
// queued at 12-28; Llama 32K-128K: 728-752 us against 767-806 static); at
// 2 per CU it lost 9 % (Qwen 1K-32K), at 8 per CU -1 to +7 %.
constexpr int64_t kQueuePlanSegmentsPerCu = 4;

// Shares per unit of a steal-scheduled call: the largest divisor d of
// num_splits with at most one workgroup per compute unit (units * d <= cus)
// and num_splits / d - 1 steal slots per share in 1..kStealMaxCap; 0 if
// none (the call then runs the static schedule).
int steal_shares_per_unit(int units, int num_splits, int cus) {
  for (int d = num_splits / 2; d >= 1; --d) {
    if (num_splits % d != 0) continue;
    const int cap = num_splits / d - 1;
    if (cap < 1 || cap > fd::kStealMaxCap) continue;
    if ((int64_t)units * d > cus) continue;
    if ((int64_t)units * d > fd::kStealMaxShares) continue;
    return d;
  }
  return 0;
}

int launch_split(const void* q, const void* k, const void* v, const int32_t* cu, int batch,
                 int heads, int kv_heads, int dim, int num_splits, float scale, Format fmt,
                 const Workspace& w, void* out, int direct, hipStream_t stream, int dtype,
                 const fd_kv_layout& L, const Sizes& sz, int path, int sched,
                 bool fused = false) {
  fd::SplitArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.cu = cu;
  a.opart = w.opart;
  a.lse = w.lse;
  a.mbuf = w.mbuf;
  a.lbuf = w.lbuf;
  a.out = out;
  a.sb = L.batch_stride;
  a.sh = L.head_stride;
  a.st = L.token_stride;
  a.scu = L.cu_stride;
  a.batch = batch;
  a.heads = heads;
  a.kv_heads = kv_heads;
  a.group = sz.group;
  a.num_splits = num_splits;
  a.row_chunks = sz.row_chunks;
  a.rows_per_pass = sz.rows;
  a.direct = direct;
  a.ceil_bounds = fmt == kUnnorm ? 1 : 0;
  a.unnorm = fmt == kUnnorm ? 1 : 0;
  a.scale_log2 = (float)((double)scale * kLog2e);
  // Non-temporal K/V loads pay off once the launch fills every compute unit
  // (measured; below that each workgroup's stream is latency-bound and they
  // slow it). The unpacked comparison path re-reads K/V once per query head
  // and keeps the default policy, under which those re-reads can hit cache.
  int cus = 0;
  const int cst = device_cus(&cus);
  if (cst != FD_OK) return cst;
  a.kv_nt = path != FD_PATH_UNPACKED && sz.workgroups >= cus ? 1 : 0;
  a.wide = sz.workgroups < cus ? 1 : 0;
  a.cus = cus;
  a.items = (int)sz.workgroups;
  // (queued launches fill the device, so they always take non-temporal loads)
  a.arrivals = fused ? w.arrivals : nullptr;
  a.queue = !fused && w.queue != nullptr && a.kv_nt && use_queue(sched) ? w.queue
                                                                                   : nullptr;
  dim3 grid((unsigned)sz.workgroups);
  const bool mfma = path == FD_PATH_MFMA || (path == FD_PATH_AUTO && auto_mfma(dtype, dim, sz.group));
  // Steal schedule: whole calls in the normalised format on the
  // matrix-core kernel; one workgroup per share, non-temporal loads.
  a.steal = nullptr;
  a.steal_nsh = a.steal_cap = a.steal_chunks = a.steal_shares = 0;
  if (sched == FD_SCHED_STEAL && !fused && !direct && fmt == kNormalised && mfma && dim == 128 &&
      w.steal != nullptr) {
    const int units = batch * kv_heads * sz.row_chunks;
    const int d = steal_shares_per_unit(units, num_splits, cus);
    if (d > 0) {
      a.steal = w.steal;
      a.steal_nsh = d;
      a.steal_cap = num_splits / d - 1;
      a.steal_chunks = kStealChunks;
      a.steal_shares = units * d;
      a.queue = nullptr;
      a.kv_nt = 1;
      a.wide = 0;
      grid = dim3((unsigned)a.steal_shares);
      const hipError_t er = fd::launch_steal_reset(a.steal, a.steal_shares, stream);
      if (er != hipSuccess) return hip_fail(er, "steal reset launch");
    }
  }
  if (a.queue != nullptr) {
    const hipError_t er = fd::launch_queue_reset(a.queue, stream);
    if (er != hipSuccess) return hip_fail(er, "queue reset launch");
  }
  hipError_t e;
  switch (dtype) {
    case FD_F32: e = fd::launch_split_f32(a, dim, sz.rows, mfma, grid, stream); break;
    case FD_F16: e = fd::launch_split_f16(a, dim, sz.rows, mfma, grid, stream); break;
    default: e = fd::launch_split_bf16(a, dim, sz.rows, mfma, grid, stream); break;
  }
  if (e != hipSuccess) return hip_fail(e, "split kernel launch");
  return FD_OK;
}

int split_impl(Format fmt, const void* q, const void* k, const void* v,
               const int32_t* cu_seqlens_k, int batch, int heads, int kv_heads, int dim,
               int num_splits, float scale, void* workspace, void* stream, int dtype,
               const fd_kv_layout* layout, int sched) {
  const int path = g_path;
  Sizes sz;
  int st = check_common(batch, heads, kv_heads, dim, num_splits, dtype, &sz, rows_per_pass(path));
  if (st != FD_OK) return st;
  if (!q || !k || !v || !cu_seqlens_k || !workspace) return FD_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(workspace))
    return FD_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return FD_ERR_INVALID_ARG;
  fd_kv_layout L;
  st = check_layout(layout, kv_heads, dim, dtype, &L);
  if (st != FD_OK) return st;
  const Workspace w = workspace_views(fmt, workspace, batch, heads, dim, num_splits);
  return launch_split(q, k, v, cu_seqlens_k, batch, heads, kv_heads, dim, num_splits, scale, fmt,
                      w, nullptr, 0, static_cast<hipStream_t>(stream), dtype, L, sz, path,
                      sched);
}

int combine_impl(Format fmt, const void* workspace, int batch, int heads, int dim,
                 int num_splits, void* out, void* stream, int dtype) {
  if (batch < 1 || heads < 1 || num_splits < 1 || num_splits > FD_MAX_SPLITS)
    return FD_ERR_INVALID_ARG;
  if ((int64_t)batch * heads > INT_MAX / 2) return FD_ERR_INVALID_ARG;
  if (dtype != FD_F32 && dtype != FD_F16 && dtype != FD_BF16) return FD_ERR_UNSUPPORTED;
  if (!dim_ok(dim)) return FD_ERR_UNSUPPORTED;
  if (!workspace || !out || !aligned16(workspace) || !aligned16(out)) return FD_ERR_INVALID_ARG;
  const Workspace w =
      workspace_views(fmt, const_cast<void*>(workspace), batch, heads, dim, num_splits);
  fd::CombineArgs a;
  a.opart = w.opart;
  a.lse = w.lse;
  a.mbuf = w.mbuf;
  a.lbuf = w.lbuf;
  a.out = out;
  a.batch = batch;
  a.heads = heads;
  a.num_splits = num_splits;
  a.unnorm = fmt == kUnnorm ? 1 : 0;
  hipError_t e = fd::launch_combine(a, dtype, dim, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "combine kernel launch");
  return FD_OK;
}

// Checks of a whole-call entry point other than its workspace.
int check_attention(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_k,
                    int batch, int heads, int kv_heads, int dim, int num_splits, float scale,
                    const void* out, int dtype, const fd_kv_layout* layout, int path, Sizes* sz,
                    fd_kv_layout* L) {
  int st = check_common(batch, heads, kv_heads, dim, num_splits, dtype, sz, rows_per_pass(path));
  if (st != FD_OK) return st;
  if (!q || !k || !v || !cu_seqlens_k || !out) return FD_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return FD_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return FD_ERR_INVALID_ARG;
  return check_layout(layout, kv_heads, dim, dtype, L);
}

int attention_impl(Format fmt, const void* q, const void* k, const void* v,
                   const int32_t* cu_seqlens_k, int batch, int heads, int kv_heads, int dim,
                   int num_splits, float scale, void* out, void* workspace, void* stream,
                   int dtype, const fd_kv_layout* layout, int combine) {
  const int path = g_path;
  Sizes sz;
  fd_kv_layout L;
  int st = check_attention(q, k, v, cu_seqlens_k, batch, heads, kv_heads, dim, num_splits, scale,
                           out, dtype, layout, path, &sz, &L);
  if (st != FD_OK) return st;
  if (num_splits > 1 && !workspace) return FD_ERR_INVALID_ARG;
  if (workspace && !aligned16(workspace)) return FD_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (num_splits == 1) {
    // one split is the whole sequence under either bound rule: one launch
    Workspace w;
    if (workspace != nullptr && fmt == kNormalised)
      w.queue = workspace_views(fmt, workspace, batch, heads, dim, 1).queue;
    return launch_split(q, k, v, cu_seqlens_k, batch, heads, kv_heads, dim, 1, scale, fmt, w, out,
                        1, s, dtype, L, sz, path, g_sched);
  }
  if (fmt == kNormalised && combine == FD_COMBINE_FUSED) {
    // one launch: the split kernel's last workgroup per unit merges
    const Workspace w = workspace_views(fmt, workspace, batch, heads, dim, num_splits);
    return launch_split(q, k, v, cu_seqlens_k, batch, heads, kv_heads, dim, num_splits, scale,
                        fmt, w, out, 0, s, dtype, L, sz, path, FD_SCHED_STATIC, true);
  }
  st = split_impl(fmt, q, k, v, cu_seqlens_k, batch, heads, kv_heads, dim, num_splits, scale,
                  workspace, stream, dtype, layout, g_sched);
  if (st != FD_OK) return st;
  return combine_impl(fmt, workspace, batch, heads, dim, num_splits, out, stream, dtype);
}

// Modelled time (us) of a call with ns splits (see the model above). With
// unequal lengths, workgroups are handed out as compute units free up, which
// finishes within the average load plus the largest workgroup
// (list-scheduling bound), at the rate of min(CUs, workgroups) at once.
double model_call_us(int64_t units, int64_t ns, int cus, double key_bytes, int64_t max_len,
                     double all_bytes, bool uniform, double partial_bytes) {
  const int64_t wgs = units * ns;
  const double wg_bytes = std::ceil((double)max_len / (double)ns) * key_bytes;
  auto per_byte = [](double n) {
    return 1.0 / kModelRateBytesPerUs + n / kModelContentionBytesPerUs;
  };
  double t = kModelLaunchUs;
  if (uniform) {
    for (int64_t rem = wgs; rem > 0;) {
      const int64_t n = rem < cus ? rem : cus;
      t += kModelWorkgroupUs + wg_bytes * per_byte((double)n);
      rem -= n;
    }
  } else {
    const double n = (double)(wgs < cus ? wgs : cus);
    const double rounds = std::ceil((double)wgs / (double)cus);
    t += rounds * kModelWorkgroupUs + (all_bytes / n + wg_bytes) * per_byte(n);
  }
  if (ns > 1) t += kModelCombineUs + kModelCombineUsPerMB * partial_bytes * 1e-6;
  return t;
}

struct PlanInputs {
  Sizes sz;
  int64_t min_len, max_len, units;
  double key_bytes, all_bytes, partial_bytes_per_split;
  int cus;
};

int plan_inputs(int batch, int heads, int kv_heads, int dim, int dtype,
                const int32_t* seqlens_host, int num_cus, PlanInputs* p) {
  if (seqlens_host == nullptr) return FD_ERR_INVALID_ARG;
  int st = check_common(batch, heads, kv_heads, dim, 1, dtype, &p->sz);
  if (st != FD_OK) return st;
  int64_t min_len = INT64_MAX, max_len = 0;
  double total_keys = 0.0;
  for (int b = 0; b < batch; ++b) {
    const int64_t x = seqlens_host[b];
    if (x < min_len) min_len = x;
    if (x > max_len) max_len = x;
    total_keys += (double)x;
  }
  if (min_len < 1) return FD_ERR_EMPTY_SPLIT;
  if (num_cus < 0) return FD_ERR_INVALID_ARG;
  if (num_cus == 0) {
    st = device_cus(&num_cus);
    if (st != FD_OK) return st;
  }
  p->min_len = min_len;
  p->max_len = max_len;
  p->units = (int64_t)batch * kv_heads * p->sz.row_chunks;
  p->key_bytes = 2.0 * dim * (dtype == FD_F32 ? 4 : 2);  // one K + one V row
  p->all_bytes = total_keys * (double)kv_heads * p->sz.row_chunks * p->key_bytes;
  p->partial_bytes_per_split = (double)batch * heads * (dim + 1) * 4.0;
  p->cus = num_cus;
  return FD_OK;
}

// The static plan: among split counts that leave every split non-empty,
// keep >= kPlanMinKeysPerSplit keys per split of the longest sequence and
// a bounded workgroup count, the least modelled time; ties to fewer
// splits. Launches of fewer workgroups than compute units are priced by
// the same rounds (one round), which is the wave quantisation of
// 04_flash_decoding.py demo 4 against the device's compute units.
int plan_static_splits(const PlanInputs& p, int max_splits) {
  int64_t cap = (p.max_len + kPlanMinKeysPerSplit - 1) / kPlanMinKeysPerSplit;
  if (cap > p.min_len) cap = p.min_len;
  if (cap > max_splits) cap = max_splits;
  while (cap > 1 && p.units * cap > kMaxWorkgroups) --cap;
  if (cap < 1) cap = 1;
  double best = 0.0;
  int choice = 1;
  for (int64_t ns = 1; ns <= cap; ++ns) {
    const double t = model_call_us(p.units, ns, p.cus, p.key_bytes, p.max_len, p.all_bytes,
                                   p.min_len == p.max_len, p.partial_bytes_per_split * ns);
    if (ns == 1 || t < best) {
      best = t;
      choice = (int)ns;
    }
  }
  return choice;
}

// The steal layout's partial-slot count for a planned batch: as many
// shares per unit as fit one per compute unit, each with kStealPlanCap
// steal slots; 0 where the steal schedule cannot run (not the matrix-core
// kernel, head dim other than 128), the slots exceed max_splits or the
// words, or a share of the longest sequence would have fewer than two
// chunks.
int steal_plan_slots(const PlanInputs& p, int dim, int dtype, int max_splits) {
  const bool mfma = g_path == FD_PATH_MFMA ||
                    (g_path == FD_PATH_AUTO && auto_mfma(dtype, dim, p.sz.group));
  if (!mfma || dim != 128) return 0;
  const int64_t nsh = p.units < p.cus ? p.cus / p.units : 1;
  const int64_t slots = nsh * (1 + kStealPlanCap);
  if (slots > max_splits || p.units * nsh > fd::kStealMaxShares ||
      p.max_len / nsh < 2 * fd::kStealMinChunk)
    return 0;
  return (int)slots;
}

}  // namespace

extern "C" {

size_t fd_workspace_bytes(int batch, int heads, int num_splits, int dim) {
  if (batch < 1 || heads < 1 || num_splits < 1 || num_splits > FD_MAX_SPLITS || !dim_ok(dim))
    return 0;
  const double est = (double)batch * heads * num_splits * (dim + 2) * 4.0;
  if (est > 1e18) return 0;
  return workspace_bytes(kNormalised, batch, heads, dim, num_splits);
}

size_t fd_workspace_bytes_unnorm(int batch, int heads, int num_splits, int dim) {
  if (batch < 1 || heads < 1 || num_splits < 1 || num_splits > FD_MAX_SPLITS || !dim_ok(dim))
    return 0;
  const double est = (double)batch * heads * num_splits * (dim + 2) * 4.0;
  if (est > 1e18) return 0;
  return workspace_bytes(kUnnorm, batch, heads, dim, num_splits);
}

int fd_plan_splits(int batch, int heads, int kv_heads, int dim, int dtype,
                   const int32_t* seqlens_host, int num_cus, int max_splits,
                   int* num_splits_out) {
  if (num_splits_out == nullptr) return FD_ERR_INVALID_ARG;
  PlanInputs p;
  const int st = plan_inputs(batch, heads, kv_heads, dim, dtype, seqlens_host, num_cus, &p);
  if (st != FD_OK) return st;
  if (max_splits <= 0 || max_splits > FD_MAX_SPLITS) max_splits = FD_MAX_SPLITS;
  // Under the steal schedule, a call that can take it gets the steal
  // layout (steal_plan_slots); otherwise the least modelled time.
  const int slots = g_sched == FD_SCHED_STEAL ? steal_plan_slots(p, dim, dtype, max_splits) : 0;
  *num_splits_out = slots > 0 ? slots : plan_static_splits(p, max_splits);
  return FD_OK;
}

int fd_plan_schedule(int batch, int heads, int kv_heads, int dim, int dtype,
                     const int32_t* seqlens_host, int num_cus, int max_splits,
                     int* schedule_out, int* num_splits_out) {
  if (schedule_out == nullptr || num_splits_out == nullptr) return FD_ERR_INVALID_ARG;
  PlanInputs p;
  const int st = plan_inputs(batch, heads, kv_heads, dim, dtype, seqlens_host, num_cus, &p);
  if (st != FD_OK) return st;
  if (max_splits <= 0 || max_splits > FD_MAX_SPLITS) max_splits = FD_MAX_SPLITS;
  // Ragged batches: the queue schedule at about kQueuePlanSegmentsPerCu
  // segments per compute unit (never more splits than the shortest
  // sequence has keys, nor fewer than 256 keys per split of the longest).
  if (2 * p.max_len >= 3 * p.min_len) {
    int64_t ns = (kQueuePlanSegmentsPerCu * (int64_t)p.cus + p.units / 2) / p.units;
    const int64_t keys_cap = (p.max_len + kPlanMinKeysPerSplit - 1) / kPlanMinKeysPerSplit;
    if (ns > keys_cap) ns = keys_cap;
    if (ns > p.min_len) ns = p.min_len;
    if (ns > max_splits) ns = max_splits;
    while (ns > 1 && p.units * ns > kMaxWorkgroups) --ns;
    if (ns < 1) ns = 1;
    // the queue runs only where the launch fills the device
    if (p.units * ns >= p.cus) {
      *schedule_out = FD_SCHED_QUEUE;
      *num_splits_out = (int)ns;
      return FD_OK;
    }
  }
  // Near-uniform batches: the steal schedule where it measured faster: a
  // layout exists, the lengths lie within a factor of kStealPlanMaxRatio of
  // each other, and each share of the longest sequence streams
  // kStealPlanMinShareBytes or more (one K and one V row of one KV head per
  // key).
  const int slots = steal_plan_slots(p, dim, dtype, max_splits);
  if (slots > 0) {
    const int64_t nsh = slots / (1 + kStealPlanCap);
    const double share_bytes = (double)(p.max_len / nsh) * p.key_bytes;
    if (p.max_len <= kStealPlanMaxRatio * p.min_len && share_bytes >= kStealPlanMinShareBytes) {
      *schedule_out = FD_SCHED_STEAL;
      *num_splits_out = slots;
      return FD_OK;
    }
  }
  *schedule_out = FD_SCHED_STATIC;
  *num_splits_out = plan_static_splits(p, max_splits);
  return FD_OK;
}

double fd_plan_time_us(int batch, int heads, int kv_heads, int dim, int dtype,
                       const int32_t* seqlens_host, int num_cus, int num_splits) {
  PlanInputs p;
  if (num_splits < 1 || num_splits > FD_MAX_SPLITS) return -1.0;
  if (plan_inputs(batch, heads, kv_heads, dim, dtype, seqlens_host, num_cus, &p) != FD_OK)
    return -1.0;
  return model_call_us(p.units, num_splits, p.cus, p.key_bytes, p.max_len, p.all_bytes,
                       p.min_len == p.max_len, p.partial_bytes_per_split * num_splits);
}

int fd_decode_split(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_k,
                    int batch, int heads, int kv_heads, int dim, int num_splits, float scale,
                    void* workspace, void* stream, int dtype, const fd_kv_layout* layout) {
  return split_impl(kNormalised, q, k, v, cu_seqlens_k, batch, heads, kv_heads, dim, num_splits,
                    scale, workspace, stream, dtype, layout, g_sched);
}

int fd_decode_combine(const void* workspace, int batch, int heads, int dim, int num_splits,
                      void* out, void* stream, int dtype) {
  return combine_impl(kNormalised, workspace, batch, heads, dim, num_splits, out, stream, dtype);
}

int fd_decode_attention(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_k,
                        int batch, int heads, int kv_heads, int dim, int num_splits, float scale,
                        void* out, void* workspace, void* stream, int dtype,
                        const fd_kv_layout* layout) {
  return attention_impl(kNormalised, q, k, v, cu_seqlens_k, batch, heads, kv_heads, dim,
                        num_splits, scale, out, workspace, stream, dtype, layout, g_combine);
}

int fd_decode_split_unnorm(const void* q, const void* k, const void* v,
                           const int32_t* cu_seqlens_k, int batch, int heads, int kv_heads,
                           int dim, int num_splits, float scale, void* workspace, void* stream,
                           int dtype, const fd_kv_layout* layout) {
  return split_impl(kUnnorm, q, k, v, cu_seqlens_k, batch, heads, kv_heads, dim, num_splits,
                    scale, workspace, stream, dtype, layout, g_sched);
}

int fd_decode_combine_unnorm(const void* workspace, int batch, int heads, int dim,
                             int num_splits, void* out, void* stream, int dtype) {
  return combine_impl(kUnnorm, workspace, batch, heads, dim, num_splits, out, stream, dtype);
}

int fd_decode_attention_unnorm(const void* q, const void* k, const void* v,
                               const int32_t* cu_seqlens_k, int batch, int heads, int kv_heads,
                               int dim, int num_splits, float scale, void* out, void* workspace,
                               void* stream, int dtype, const fd_kv_layout* layout) {
  return attention_impl(kUnnorm, q, k, v, cu_seqlens_k, batch, heads, kv_heads, dim, num_splits,
                        scale, out, workspace, stream, dtype, layout, FD_COMBINE_SEPARATE);
}

int fd_decode_attention_noalloc(const void* q, const void* k, const void* v,
                                const int32_t* cu_seqlens_k, int batch, int heads, int kv_heads,
                                int dim, int num_splits, float scale, void* out, void* stream,
                                int dtype, const fd_kv_layout* layout) {
  Sizes sz;
  fd_kv_layout L;
  const int st = check_attention(q, k, v, cu_seqlens_k, batch, heads, kv_heads, dim, num_splits,
                                 scale, out, dtype, layout, g_path, &sz, &L);
  if (st != FD_OK) return st;
  void* ws = nullptr;
  if (num_splits > 1) {
    const size_t need = workspace_bytes(kNormalised, batch, heads, dim, num_splits);
    if (need > FD_NOALLOC_SCRATCH_BYTES) {
      std::snprintf(g_last_error, sizeof(g_last_error),
                    "the partials need %zu bytes, the static scratch holds %zu", need,
                    (size_t)FD_NOALLOC_SCRATCH_BYTES);
      return FD_ERR_SCRATCH;
    }
    const int s2 = scratch_on_device(&ws);
    if (s2 != FD_OK) return s2;
  }
  // the scratch's arrival counters would move with the call's sizes, over
  // earlier calls' partials, so these calls always merge in the combine kernel
  return attention_impl(kNormalised, q, k, v, cu_seqlens_k, batch, heads, kv_heads, dim,
                        num_splits, scale, out, ws, stream, dtype, layout, FD_COMBINE_SEPARATE);
}

const char* fd_status_string(int status) {
  switch (status) {
    case FD_OK: return "ok";
    case FD_ERR_INVALID_ARG: return "invalid argument";
    case FD_ERR_UNSUPPORTED: return "unsupported configuration";
    case FD_ERR_EMPTY_SPLIT: return "a sequence has no key (empty split)";
    case FD_ERR_HIP: return "HIP runtime error";
    case FD_ERR_SCRATCH: return "the call needs more than the static scratch holds";
    default: return "unknown status";
  }
}

const char* fd_last_error(void) { return g_last_error; }

int fd_set_combine(int mode) {
  if (mode != FD_COMBINE_SEPARATE && mode != FD_COMBINE_FUSED) return -1;
  const int prev = g_combine;
  g_combine = mode;
  return prev;
}

int fd_set_schedule(int sched) {
  if (sched != FD_SCHED_AUTO && sched != FD_SCHED_STATIC && sched != FD_SCHED_QUEUE &&
      sched != FD_SCHED_STEAL)
    return -1;
  const int prev = g_sched;
  g_sched = sched;
  return prev;
}

int fd_set_kernel_path(int path) {
  if (path != FD_PATH_AUTO && path != FD_PATH_VALU && path != FD_PATH_MFMA &&
      path != FD_PATH_UNPACKED)
    return -1;
  const int prev = g_path;
  g_path = path;
  return prev;
}

}  // extern "C"
