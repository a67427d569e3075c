// Internal declarations shared by the host layer and the kernel sources of
// libfd. Not part of the public ABI (see include/fd.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fd {

constexpr int kWave = 64;          // CDNA wavefront width
#ifndef FD_WAVES_VALU
#define FD_WAVES_VALU 4
#endif
#ifndef FD_WAVES_MFMA
#define FD_WAVES_MFMA 4
#endif
// waves per split workgroup of the VALU and the matrix-core kernel
constexpr int kWavesValu = FD_WAVES_VALU;
constexpr int kWavesMfma = FD_WAVES_MFMA;
// VALU workgroups of launches with fewer workgroups than compute units,
// where each workgroup's own stream sets the time. Measured on MI355X: the
// fp32 GQA-8 case of 7 workgroups (10,000 keys, D = 128) goes from 82 to
// 66.5 us with 8 waves; full launches gain nothing (MHA D = 128 level) or
// lose (D = 16..64 13-43 % slower) with 8, and the matrix-core kernel shows
// no consistent gain at any launch size.
constexpr int kWavesValuWide = 8;
constexpr int kMaxRowsPerPass = 8; // query rows of one GQA group handled per workgroup
// Resident matrix-core split workgroups per compute unit, enforced by
// reserving LDS at launch (registers alone allow 3). Measured on MI355X:
// the varlen Qwen batch (1024 workgroups of very unequal length) runs its
// split kernel in 191 instead of 196.5 us, because its longest segments,
// which end last, get a larger share of the bandwidth; every other matrix-
// core workload measured is within 0.3 %. Launches the planner sizes to one
// pass never have more than one workgroup per CU anyway.
constexpr int kMfmaWorkgroupsPerCu = 2;
constexpr int kLdsBytesPerCu = 160 * 1024;
constexpr int kLptMaxBatch = 64;   // batches up to this size run longest sequence first
#ifndef FD_LOADS_PER_TILE
#define FD_LOADS_PER_TILE 4
#endif
// 16-byte K (and V) loads per lane per VALU tile. 16-bit rows of head dim
// <= 32 take 2: measured on MI355X (MHA, 4 x 32 heads x 4K keys) the split
// kernel goes from 11.0 to 9.6 us at D = 16 and from 14.9 to 13.6 us at
// D = 32, is level at D = 64 and 128, and fp32 launches of a few
// workgroups are 13 % slower with 2.
constexpr int kLoadsPerTile = FD_LOADS_PER_TILE;
constexpr int valu_loads_per_tile(int elem_bytes, int dim) {
  return elem_bytes == 2 && dim <= 32 ? 2 : kLoadsPerTile;
}
#ifndef FD_PREFETCH_TILES_VALU
#define FD_PREFETCH_TILES_VALU 1
#endif
#ifndef FD_PREFETCH_TILES_MFMA
#define FD_PREFETCH_TILES_MFMA 1
#endif
// Tiles whose loads are in flight while a wave computes the current one,
// for the VALU and the matrix-core split kernel.
constexpr int kPrefetchTilesValu = FD_PREFETCH_TILES_VALU;
constexpr int kPrefetchTilesMfma = FD_PREFETCH_TILES_MFMA;

// Steal schedule limits: steal slots per share (a 4-bit field of the share
// word) and share words in the workspace's control block.
constexpr int kStealMaxCap = 15;
constexpr int kStealMaxShares = 4096;
// Smallest chunk (keys) of the steal schedule: an owner's claim runs a
// whole chunk ahead of its use, so its round trip is hidden.
constexpr int kStealMinChunk = 512;

// Arguments of the split kernel (passed by value).
struct SplitArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* cu;
  float* opart;     // [B, H, ns, D] fp32 (workspace mode): o_s, or acc_s if unnorm
  float* lse;       // [B, ns, H]   fp32 (workspace mode, normalised format)
  float* mbuf;      // [B, H, ns]   fp32 (workspace mode, unnorm format): m_s
  float* lbuf;      // [B, H, ns]   fp32 (workspace mode, unnorm format): l_s
  void* out;        // [B, H, D] dtype (direct mode, ns == 1)
  int64_t sb, sh, st, scu;  // K/V strides in elements: batch, head, token, cu
  int batch, heads, kv_heads, group, num_splits, row_chunks;
  int rows_per_pass; // query rows of a group per workgroup (<= the kernel's rows)
  int kv_nt;        // 1: K/V loads with the non-temporal cache policy
  int wide;         // 1: VALU workgroups of kWavesValuWide waves (launches below one pass)
  int direct;       // 1: write out in dtype; 0: write the workspace
  int ceil_bounds;  // 1: ceil-equal split bounds; 0: proportional
  int unnorm;       // 1: workspace holds (m, l, acc); 0: (o_s, lse2_s)
  float scale_log2; // scale * log2(e)
  // Queue schedule: `queue` points at a claim counter that is zero when the
  // launch starts; workgroup w first takes segment w, then claims segments
  // gridDim.x, gridDim.x + 1, ... from the counter until `items` is reached.
  // nullptr: one segment per workgroup (the grid covers every segment).
  int* queue;
  int items;
  int cus;          // compute units of the device (sizes a queue-scheduled grid)
  // Single launch (fused combine): one arrival counter per (sequence, KV
  // head, row chunk), zero before the launch; the last of the unit's
  // num_splits workgroups to arrive merges the unit's partials into `out`
  // and sets the counter back to zero. nullptr: the combine kernel merges.
  int* arrivals;
  // Steal schedule (matrix-core kernel, whole calls in the normalised
  // format): the keys of each unit are cut into steal_nsh proportional
  // shares, one workgroup each (the grid); share r owns the partial slots
  // r * (1 + steal_cap) .. r * (1 + steal_cap) + steal_cap of its unit
  // (num_splits = steal_nsh * (1 + steal_cap)). Its workgroup streams its
  // share in chunks claimed ahead from its word in `steal` (zero at launch),
  // one partial for the run it streamed; workgroups that are done take the
  // back half of the unclaimed chunks of another share (at most steal_cap
  // times per share), one partial each. steal_chunks: chunks per share.
  // nullptr: off.
  unsigned long long* steal;
  int steal_nsh, steal_cap, steal_chunks, steal_shares;
};

struct CombineArgs {
  const float* opart;  // o_s, or acc_s (unnorm)
  const float* lse;    // [B, ns, H] (normalised format)
  const float* mbuf;   // [B, H, ns] (unnorm format)
  const float* lbuf;   // [B, H, ns] (unnorm format)
  void* out;
  int batch, heads, num_splits;
  int unnorm;
};

// Launchers (defined in fd_split_<dtype>.hip and fd_combine.hip). They
// return the hipError_t of the launch.
// `mfma` selects the matrix-core QK^T kernel where one exists (head dim
// 128); otherwise the VALU kernel runs.
hipError_t launch_split_f32(const SplitArgs& a, int dim, int rows, bool mfma, dim3 grid,
                            hipStream_t s);
hipError_t launch_split_f16(const SplitArgs& a, int dim, int rows, bool mfma, dim3 grid,
                            hipStream_t s);
hipError_t launch_split_bf16(const SplitArgs& a, int dim, int rows, bool mfma, dim3 grid,
                             hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, int dtype, int dim, hipStream_t s);
// Zeroes the claim counter of a queue-scheduled split launch (one thread).
hipError_t launch_queue_reset(int* queue, hipStream_t s);
// Zeroes the n share words of a steal-scheduled split launch.
hipError_t launch_steal_reset(unsigned long long* words, int n, hipStream_t s);

}  // namespace fd
