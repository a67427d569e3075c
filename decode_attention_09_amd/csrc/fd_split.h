// Split kernel of flash decoding for gfx950: one workgroup per
// (split, KV head, row chunk, sequence) computes, for the packed query rows
// of one GQA group, the online-softmax partial output of its KV segment and
// the segment's base-2 log-sum-exp -- or, in the format of
// "flash_decode_splitk.py" (MiniInfer), the segment's unnormalised state
// (max, sum, accumulator) over ceil-equal split bounds.
//
// Behaviour follows the split segment of gqa_decode_splitkv in
// "decode_attention_splitkv.py" (TileLang tutorial, ch. 18): varlen bounds
// from cu_seqlens_k, proportional segment [L*s/ns, L*(s+1)/ns), scores of
// keys outside the segment excluded, running max / sum in fp32 with exp2
// and the log2(e)-folded scale, epilogue o_s = acc / l and
// lse2_s = log2(l) + m. The mapping onto the hardware is this file's own:
//
//  * Lane layout. A K or V row of D elements is split into 16-byte chunks;
//    LPR = D*elem/16 consecutive lanes hold one row, so one wave-wide
//    buffer_load_dwordx4 fetches RPI = 64/LPR whole rows (fully used
//    128-byte lines). Every lane keeps the same chunk of q for each of the
//    G packed rows, so each K/V byte is read once for the whole group.
//  * QK^T: each lane dots its chunk (v_dot2 for fp16/bf16, FMA for fp32),
//    then the LPR lanes of a row sum with DPP butterflies (quad_perm,
//    row_half_mirror, row_mirror). The sum is identical in all LPR lanes,
//    which then all hold the score of their key for all G rows.
//  * Online softmax per lane group (the RPI keys rows of a load are handled
//    by different lane groups, each with its own running max), rescaling
//    lazily: the reference max only moves when a tile exceeds it by more
//    than 2^8, so rescaling is rare and p stays <= 256. The true max is
//    tracked beside it, and the end-of-segment merge rescales every lane
//    group onto it, so the written state refers to the segment's largest
//    score (the MiniInfer format stores it as m_s).
//  * PV: p for two keys is packed to fp16x2/bf16x2 and multiplied with the
//    matching pair of V elements (v_perm regroups them) by v_dot2, fp32 acc.
//  * Bounds: each tile's K/V loads go through a buffer descriptor whose
//    size ends at the last valid row of the segment, so rows past the
//    segment (or the tensor) read as zero without branches, and are then
//    masked out of the softmax.
//  * The waves of a workgroup (4; 8 for VALU launches with fewer workgroups
//    than compute units) take interleaved tiles of the segment and are
//    merged through LDS at the end (the same LSE merge as the combine).
//  * Register tile pipeline: the loads of the next kPrefetchTilesValu
//    (kPrefetchTilesMfma) tiles are in flight while the current tile is
//    computed.
//  * The matrix-core kernel (split_kernel_mfma, head dim 128, every dtype)
//    computes QK^T on v_mfma_f32_16x16x32_{f16,bf16} / v_mfma_f32_16x16x4_f32
//    with the group's query rows as the 16 MFMA columns; see its section.
//  * Schedules: one workgroup per segment; (queue instances) a grid of
//    one workgroup per compute unit whose workgroups claim further segments
//    from a counter once their first one is done (claim_next); or (steal
//    instances of the matrix-core kernel) one workgroup per share of each
//    unit, streaming its share in chunks claimed ahead and then taking the
//    unclaimed back half of other shares (steal_search).
//  * Single launch: with an arrival-counter array, the last of a unit's
//    workgroups merges the unit's partials itself (arrive_and_merge).
#pragma once

#include <climits>
#include <type_traits>

#include "fd_internal.h"
#include "fd_steal.h"

namespace fd {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef __bf16 b4_t __attribute__((ext_vector_type(4)));

enum { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

constexpr float kNegInf = -__builtin_inff();
constexpr float kLazyRescale = 8.0f;  // log2 units

template <int DT>
struct Elem {
  static constexpr int bytes = DT == DT_F32 ? 4 : 2;
};

// ---------------------------------------------------------------- lanes --
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Pairwise combine of 16-lane rows (0<->1, 2<->3) or of 32-lane halves with
// v_permlane16_swap / v_permlane32_swap: both lanes of a pair receive the
// two values in the same order, so op gives them bitwise equal results.
struct OpAdd {
  __device__ float operator()(float x, float y) const { return x + y; }
};
struct OpMax {
  __device__ float operator()(float x, float y) const { return fmaxf(x, y); }
};

template <typename Op>
__device__ __forceinline__ float rows_pair(float x, Op op) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return op(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}

template <typename Op>
__device__ __forceinline__ float halves_pair(float x, Op op) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return op(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}

// Reduce-scatter steps over the four 16-lane rows, for two values at once.
// rows_scatter(a, b): rows 0 and 2 get a summed over their row pair (0+1,
// 2+3), rows 1 and 3 get b summed over theirs. halves_scatter(a, b): the
// lower half (rows 0, 1) gets a summed over the halves (row r + row r+2),
// the upper half gets b. Applied to values x_{4j..4j+3} (rows_scatter on
// pairs, then halves_scatter on the results), row R ends with
// (x_{4j+R} of row 0 + of row 1) + (of row 2 + of row 3): the same sums,
// in the same order, as rows_pair then halves_pair on each value, with a
// quarter of the swaps and adds.
__device__ __forceinline__ float rows_scatter(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, a),
                                                  __builtin_bit_cast(uint32_t, b), false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

__device__ __forceinline__ float halves_scatter(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, a),
                                                  __builtin_bit_cast(uint32_t, b), false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// Sum over aligned groups of LPR lanes; every lane of a group gets the same
// (bitwise) result because each butterfly step adds the same two values.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (LPR >= 2) x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
  if constexpr (LPR >= 4) x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
  if constexpr (LPR >= 8) x += dpp_mov<0x141>(x);  // row_half_mirror
  if constexpr (LPR >= 16) x += dpp_mov<0x140>(x); // row_mirror
  if constexpr (LPR >= 32) x = rows_pair(x, OpAdd{});
  return x;
}

// Reduce across the 64/LPR lane groups of a wave: lanes with the same
// lane % LPR combine. Within a 16-lane row the groups are folded by DPP
// row rotations (lane i takes i + n mod 16), then rows and halves by the
// swaps. Every lane receives the reduction of its residue class.
template <int LPR, typename Op>
__device__ __forceinline__ float across_groups(float x, Op op) {
  if constexpr (LPR <= 1) x = op(x, dpp_mov<0x121>(x));  // row_ror:1
  if constexpr (LPR <= 2) x = op(x, dpp_mov<0x122>(x));  // row_ror:2
  if constexpr (LPR <= 4) x = op(x, dpp_mov<0x124>(x));  // row_ror:4
  if constexpr (LPR <= 8) x = op(x, dpp_mov<0x128>(x));  // row_ror:8
  if constexpr (LPR <= 16) x = rows_pair(x, op);
  if constexpr (LPR <= 32) x = halves_pair(x, op);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ------------------------------------------------------------- memory --
// Raw buffer descriptor over [base, base+bytes): loads at offsets past
// `bytes` return zero. Both inputs are wave-uniform by construction; the
// readfirstlanes tell the compiler so, keeping the descriptor in SGPRs.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const char* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  char* up = reinterpret_cast<char*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(up, (short)0,
                                           (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// 16-byte K/V load. NT: the non-temporal cache policy (the `nt` bit, value
// 2 of the buffer instructions' cache-policy operand on gfx950). K and V are
// read once per call; measured on MI355X, `nt` cuts the split kernel's time
// by 2-8 % once the launch fills every compute unit (e.g. 45.6 -> 41.8 us for
// 268 MB of MHA K/V in 2048 workgroups) but slows a launch of fewer
// workgroups than compute units by 8-27 %, where each workgroup's stream is
// latency-bound. The host chooses per launch.
template <bool NT>
__device__ __forceinline__ u4_t buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, NT ? 2 : 0));
}

// Element w of a 4-word vector, copied out by value. (__builtin_bit_cast
// applied directly to an ext_vector element reads element 0 with this
// compiler, so every reinterpretation goes through this copy.)
__device__ __forceinline__ uint32_t word(const u4_t& v, int w) {
  const uint32_t x = v[w];
  return x;
}

// ------------------------------------------------------------ numerics --
// Partial dot product of one 16-byte chunk of q with the same chunk of k.
template <int DT>
__device__ __forceinline__ float chunk_dot(const u4_t& q, const u4_t& k, float acc) {
  if constexpr (DT == DT_F16) {
#pragma unroll
    for (int w = 0; w < 4; ++w)
      acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, word(q, w)), __builtin_bit_cast(h2_t, word(k, w)),
                                   acc, false);
  } else if constexpr (DT == DT_BF16) {
#pragma unroll
    for (int w = 0; w < 4; ++w)
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2_t, word(q, w)),
                                            __builtin_bit_cast(b2_t, word(k, w)), acc, false);
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w)
      acc = __builtin_fmaf(__builtin_bit_cast(float, word(q, w)), __builtin_bit_cast(float, word(k, w)), acc);
  }
  return acc;
}

// Two fp32 probabilities -> one packed 16-bit pair (round to nearest even).
template <int DT>
__device__ __forceinline__ uint32_t pack_pair(float lo, float hi) {
  if constexpr (DT == DT_F16) {
    h2_t h = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, h);
  } else {
    b2_t h = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, h);
  }
}

template <int DT>
__device__ __forceinline__ float pair_dot(uint32_t p, uint32_t v, float acc) {
  if constexpr (DT == DT_F16)
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, p), __builtin_bit_cast(h2_t, v), acc,
                                  false);
  else
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2_t, p),
                                           __builtin_bit_cast(b2_t, v), acc, false);
}

template <int DT>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float x) {
  if constexpr (DT == DT_F32)
    static_cast<float*>(out)[idx] = x;
  else if constexpr (DT == DT_F16)
    static_cast<_Float16*>(out)[idx] = (_Float16)x;
  else
    static_cast<__bf16*>(out)[idx] = (__bf16)x;
}

// Four consecutive output elements (the index is a multiple of 4).
template <int DT>
__device__ __forceinline__ void store_out4(void* out, int64_t idx, const float (&x)[4]) {
  if constexpr (DT == DT_F32) {
    *reinterpret_cast<f4_t*>(static_cast<float*>(out) + idx) = f4_t{x[0], x[1], x[2], x[3]};
  } else if constexpr (DT == DT_F16) {
    *reinterpret_cast<h4_t*>(static_cast<_Float16*>(out) + idx) =
        h4_t{(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]};
  } else {
    *reinterpret_cast<b4_t*>(static_cast<__bf16*>(out) + idx) =
        b4_t{(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};
  }
}

// ------------------------------------------------------- work decoding --
// One workgroup per segment ("item"): workgroup -> (split, KV head, row
// chunk, sequence rank), split index fastest, without memory access; then
// the sequence, its varlen bounds and the proportional segment.
//
// Workgroups are dispatched roughly in index order, so for batches of up to
// kLptMaxBatch sequences rank r is the r-th longest sequence (ties by
// index): long segments start first and short ones fill the tail
// (longest-processing-time order). With equal lengths the order is the
// identity, so a workgroup loads its q rows for sequence `rank` while
// cu_seqlens_k is in flight and reloads them only in a varlen batch.
struct WorkItem {
  int sid, kvh, rank, h0, nrows;
};

template <int GC>
__device__ __forceinline__ WorkItem decode_item(const SplitArgs& a, int item) {
  WorkItem w;
  w.sid = item % a.num_splits;
  item /= a.num_splits;
  const int hcn = a.kv_heads * a.row_chunks;
  const int hc = item % hcn;
  w.rank = item / hcn;
  w.kvh = hc / a.row_chunks;
  const int chunk = hc % a.row_chunks;
  w.h0 = w.kvh * a.group + chunk * a.rows_per_pass;
  w.nrows = min(GC, a.group - chunk * a.rows_per_pass);
  return w;
}

// Per-lane view of cu_seqlens_k for batches of up to kLptMaxBatch
// sequences, one load per lane: lane l < batch holds cu[l], cu[l+1] and the
// LPT rank of sequence l (lanes past the batch: rank -1). Each wave ranks
// the lengths itself; an all-equal batch skips the ranking.
struct LaneSeqs {
  int lo, hi, rank;
};

// cu_seqlens_k and the batch size. The split kernels take them as their
// first two arguments, ahead of SplitArgs, so that they are preloaded into
// SGPRs at wave launch (the library is built with
// -amdgpu-kernarg-preload-count=2): the cu_seqlens_k load then starts at
// once and overlaps the fetch of the other arguments, instead of waiting
// for it (two dependent memory round trips before the first K/V load).
struct SeqTable {
  const int32_t* cu;
  int batch;
};

__device__ __forceinline__ LaneSeqs lane_seqs(const SeqTable& a) {
  LaneSeqs s{0, 0, -1};
  if (a.batch > kLptMaxBatch) return s;
  const int lane = threadIdx.x & (kWave - 1);
  const bool mine = lane < a.batch;
  if (mine) {
    s.lo = a.cu[lane];
    s.hi = a.cu[lane + 1];
  }
  const int len = mine ? s.hi - s.lo : -1;
  const int len0 = __builtin_amdgcn_readfirstlane(len);
  if (__builtin_amdgcn_ballot_w64(mine && len != len0) == 0) {
    s.rank = mine ? lane : -1;
    return s;
  }
  int rank = 0;
  for (int j = 0; j < a.batch; ++j) {
    const int lj = __builtin_amdgcn_readlane(len, j);
    rank += (lj > len || (lj == len && j < lane)) ? 1 : 0;
  }
  s.rank = mine ? rank : -1;
  return s;
}

struct Segment {
  int b, sid, kvh, h0, nrows;
  int64_t nkeys;
  const char* k;   // first K row of the segment
  const char* v;   // first V row of the segment
  uint32_t tsb;    // bytes between consecutive keys
};

// The sequence of an item (b) and its cu_seqlens_k bounds.
__device__ __forceinline__ void sequence_of(const SeqTable& st, const WorkItem& w,
                                            const LaneSeqs& ls, int& b, int& cu0, int& cu1) {
  if (st.batch <= kLptMaxBatch) {
    const uint64_t hit = __builtin_amdgcn_ballot_w64(ls.rank == w.rank);
    b = hit ? (int)__builtin_ctzll(hit) : w.rank;
    cu0 = __builtin_amdgcn_readlane(ls.lo, b);
    cu1 = __builtin_amdgcn_readlane(ls.hi, b);
  } else {
    b = w.rank;
    cu0 = st.cu[b];
    cu1 = st.cu[b + 1];
  }
}

// Keys [seg0, seg1) of sequence b (first key row cu0) for an item.
template <int EB>
__device__ __forceinline__ Segment segment_at(const SplitArgs& a, const WorkItem& w, int b,
                                              int cu0, int64_t seg0, int64_t seg1) {
  Segment g;
  g.b = b;
  g.sid = w.sid;
  g.kvh = w.kvh;
  g.h0 = w.h0;
  g.nrows = w.nrows;
  g.nkeys = seg1 - seg0;
  const int64_t row0 =
      (int64_t)g.b * a.sb + (int64_t)cu0 * a.scu + (int64_t)g.kvh * a.sh + seg0 * a.st;
  g.k = static_cast<const char*>(a.k) + row0 * EB;
  g.v = static_cast<const char*>(a.v) + row0 * EB;
  g.tsb = (uint32_t)(a.st * EB);
  return g;
}

// The sequence, its varlen bounds and the proportional segment
// [L*s/ns, L*(s+1)/ns) (64-bit products) of an item.
template <int EB>
__device__ __forceinline__ Segment locate_segment(const SplitArgs& a, const SeqTable& st,
                                                  const WorkItem& w, const LaneSeqs& ls) {
  int b, cu0, cu1;
  sequence_of(st, w, ls, b, cu0, cu1);
  const int ns = a.num_splits;
  const int64_t L = cu1 > cu0 ? (int64_t)cu1 - cu0 : 0;
  const int sid = w.sid;
  int64_t seg0, seg1;
  if (a.ceil_bounds) {
    // ceil-equal: size = ceil(L/ns) from sid*size, cut at L (may be empty)
    const int64_t size = (L + ns - 1) / ns;
    seg0 = min(size * sid, L);
    seg1 = min(size * sid + size, L);
  } else {
    seg0 = L * sid / ns;
    seg1 = L * (sid + 1) / ns;
  }
  return segment_at<EB>(a, w, b, cu0, seg0, seg1);
}

// Descriptors for tile j of TK keys of a segment: sized to end at the last
// valid row, empty for a tile past the segment (its loads return zeros).
template <int TK, int ROWB>
__device__ __forceinline__ void tile_rsrc(const Segment& sg, int j, __amdgpu_buffer_rsrc_t& rk,
                                          __amdgpu_buffer_rsrc_t& rv) {
  const int64_t k0 = (int64_t)j * TK;
  const int64_t nv = sg.nkeys - k0;
  const uint32_t rec = nv > 0 ? (uint32_t)((min(nv, (int64_t)TK) - 1) * sg.tsb + ROWB) : 0u;
  const int64_t off = nv > 0 ? k0 * sg.tsb : 0;
  rk = make_rsrc(sg.k + off, rec);
  rv = make_rsrc(sg.v + off, rec);
}

// Merge the per-wave states (max, sum, unnormalised acc) left in LDS and
// write the split epilogue: o_s = acc / l and lse2_s = log2(l) + m, or the
// unnormalised state (m_s, l_s, acc_s) of the MiniInfer format (m_s the
// split's largest base-2 score), or the final output in dtype when the call
// has a single split. Each thread takes four consecutive dims of one row
// (one 16-byte LDS read per wave state, one vector store), so a group of 8
// rows at D = 128 is written by 256 threads in one pass.
template <int DT, int D, int GC, int NW>
__device__ __forceinline__ void store_segment(const SplitArgs& a, const Segment& sg,
                                              const float (&sm_m)[NW][GC],
                                              const float (&sm_l)[NW][GC],
                                              const float (&sm_acc)[NW][GC][D]) {
  constexpr int Q = D / 4;  // groups of four dims per row
  const int ns = a.num_splits;
  for (int idx = threadIdx.x; idx < sg.nrows * Q; idx += NW * kWave) {
    const int g = idx / Q;
    const int d = (idx % Q) * 4;
    float M = sm_m[0][g];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, sm_m[w][g]);
    float lsum = 0.0f;
    float o[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = sm_m[w][g] == kNegInf ? 0.0f : fast_exp2(sm_m[w][g] - M);
      lsum += f * sm_l[w][g];
      const f4_t x = *reinterpret_cast<const f4_t*>(&sm_acc[w][g][d]);
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] += f * x[e];
    }
    const bool any = lsum > 0.0f;
    const int h = sg.h0 + g;
    const int64_t row = ((int64_t)sg.b * a.heads + h) * ns + sg.sid;  // [B, H, ns]
    if (a.unnorm && !a.direct) {
      *reinterpret_cast<f4_t*>(a.opart + row * D + d) = f4_t{o[0], o[1], o[2], o[3]};
      if (d == 0) {
        a.mbuf[row] = M;  // -inf for an empty split
        a.lbuf[row] = lsum;
      }
      continue;
    }
    float r[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = any ? o[e] / lsum : 0.0f;
    if (a.direct) {
      store_out4<DT>(a.out, ((int64_t)sg.b * a.heads + h) * D + d, r);
    } else {
      if (a.arrivals != nullptr) {
        // fused launch: agent-scope (write-through) stores, which the last
        // workgroup of the unit reads after the release/acquire on the
        // arrival counter. Measured on MI355X against plain stores (whose
        // lines the release then writes back from L2): flash-decoding B8/8K
        // 26.2 -> 21.1 us and B1/64K 37.8 -> 33.2 us per call.
#pragma unroll
        for (int e = 0; e < 4; ++e)
          __hip_atomic_store(a.opart + row * D + d + e, r[e], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        if (d == 0)
          __hip_atomic_store(a.lse + ((int64_t)sg.b * ns + sg.sid) * a.heads + h,
                             any ? fast_log2(lsum) + M : kNegInf, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        continue;
      }
      *reinterpret_cast<f4_t*>(a.opart + row * D + d) = f4_t{r[0], r[1], r[2], r[3]};
      if (d == 0)
        a.lse[((int64_t)sg.b * ns + sg.sid) * a.heads + h] = any ? fast_log2(lsum) + M : kNegInf;
    }
  }
}

// ------------------------------------------------ single-launch combine --
// In a fused launch, a workgroup counts itself in at its unit's arrival
// counter once its partials are stored; the last of the unit's num_splits
// workgroups merges the unit's partials into `out` -- the combine segment
// of gqa_decode_splitkv in "decode_attention_splitkv.py" (TileLang tutorial,
// ch. 18) and the merge of "04_flash_decoding.py" (CS349E lecture 11),
// demo 1: M = max_s lse_s, lse = M + log2 sum_s 2^(lse_s - M),
// o = sum_s 2^(lse_s - lse) o_s -- and sets the counter back to zero.
// Synchronisation follows the HIP memory model at agent scope: the barrier
// orders every thread's partial stores before thread 0's acq_rel fetch_add,
// whose release makes them visible to the workgroup that later acquires
// the counter; that last arriver's fetch_add plus an acquire fence in each
// of its waves make every other workgroup's partials visible to its loads.
// All threads of the workgroup call it (it synchronises); `slot` is an LDS
// int for the broadcast.
template <int DT, int D, int NW>
__device__ __forceinline__ void arrive_and_merge(const SplitArgs& a, const Segment& sg, int unit,
                                                 int& slot) {
  __syncthreads();
  if (threadIdx.x == 0)
    slot = __hip_atomic_fetch_add(a.arrivals + unit, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (slot != a.num_splits - 1) return;  // uniform: a split of this unit is still running
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  constexpr int Q = D / 4;  // groups of four dims per row, as in store_segment
  const int ns = a.num_splits;
  const int64_t kst = a.heads;  // LSE [B, ns, H]: split stride
  for (int idx = threadIdx.x; idx < sg.nrows * Q; idx += NW * kWave) {
    const int g = idx / Q;
    const int d = (idx % Q) * 4;
    const int h = sg.h0 + g;
    const float* lse = a.lse + (int64_t)sg.b * ns * a.heads + h;
    const float* op = a.opart + ((int64_t)sg.b * a.heads + h) * ns * D + d;  // split stride: D
    float M = kNegInf;
#pragma unroll 8
    for (int s = 0; s < ns; ++s) M = fmaxf(M, lse[s * kst]);
    float o[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (M != kNegInf) {  // all splits empty -> zero row
      float tot = 0.0f;
#pragma unroll 8
      for (int s = 0; s < ns; ++s) tot += fast_exp2(lse[s * kst] - M);
      const float lse_all = M + fast_log2(tot);
#pragma unroll 8
      for (int s = 0; s < ns; ++s) {
        const float w = fast_exp2(lse[s * kst] - lse_all);
        const f4_t x = *reinterpret_cast<const f4_t*>(op + (int64_t)s * D);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = __builtin_fmaf(w, x[e], o[e]);
      }
    }
    store_out4<DT>(a.out, ((int64_t)sg.b * a.heads + h) * D + d, o);
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(a.arrivals + unit, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Queue schedule: after a segment, thread 0 claims the next one from the
// counter (segments below gridDim.x are the workgroups' first ones, taken
// without a claim). The barrier hands the index to every thread and keeps the
// next segment's LDS writes behind all reads of this one. A relaxed atomic
// suffices: the counter passes no data, each value goes to exactly one
// claim, and the partials are read only by the next launch.
__device__ __forceinline__ int claim_next(const SplitArgs& a, int& slot) {
  if (threadIdx.x == 0)
    slot = (int)gridDim.x +
           __hip_atomic_fetch_add(a.queue, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  return slot;
}

// ------------------------------------------------------ steal schedule --
// Work stealing at chunk granularity for launches whose workgroups stream
// equal amounts at unequal rates (on MI355X the XCDs of one launch finish
// their equal segments up to 20 % apart, and workgroups on one XCD differ
// too). Share r of a unit is the proportional key range
// [L*r/nsh, L*(r+1)/nsh), cut into nc chunks of ck keys (the last one
// shorter). Its workgroup (the owner) streams chunk 0 at once and claims
// chunks 1, 2, ... one at a time, each claim issued a chunk ahead, so its
// run [0, n) is one contiguous stream with one partial. A workgroup whose
// run is over takes, from the share with the most unclaimed chunks, the
// back half of them, rounded up (a thief's run, one partial in the next
// steal slot of that share). Each chunk goes to exactly one run: both
// sides update the share's word with one atomic operation, the owner from
// the front and a thief from the back; an owner's claim succeeds only below
// the back count of the word value it replaces, a take only covers chunks
// above the front count of the value it replaces, so whichever comes first
// bounds the other. The owner claims until a claim fails, so the front and
// back runs meet. Nobody waits for another workgroup: a claim or a take
// that finds nothing ends that part of the walk.
//
// The share word and the arithmetic of claims and takes are in fd_steal.h.
constexpr int kStealKeyQuantum = 64;       // chunk keys: a multiple of one tile per wave
constexpr int kStealScans = 64;            // victim searches per workgroup, at most

// Schedules of the matrix-core kernel (template argument).
constexpr int kSchedStatic = 0, kSchedQueue = 1, kSchedSteal = 2;

struct Share {
  int64_t start, len, ck;  // first key, keys, keys per chunk
  int nc;                  // chunks (>= 1)
};

// Share r of nsh of a sequence of L keys, in about `chunks` chunks of a
// multiple of kStealKeyQuantum keys (at most `chunks`, which the host keeps
// below 2^20 - 2, so the word's fields cannot overflow).
__device__ __forceinline__ Share share_of(int64_t L, int r, int nsh, int chunks) {
  Share s;
  s.start = L * r / nsh;
  s.len = L * (r + 1) / nsh - s.start;
  const int64_t per = (s.len + chunks - 1) / chunks;
  s.ck = (per + kStealKeyQuantum - 1) / kStealKeyQuantum * kStealKeyQuantum;
  if (s.ck < kStealMinChunk) s.ck = kStealMinChunk;
  const int64_t n = (s.len + s.ck - 1) / s.ck;
  s.nc = n > 0 ? (int)n : 1;
  return s;
}

// A slot of no run: zero output and LSE -inf (ignored by the merge).
template <int D, int NW>
__device__ __forceinline__ void store_empty(const SplitArgs& a, const Segment& sg, int sid) {
  constexpr int Q = D / 4;
  const int ns = a.num_splits;
  for (int idx = threadIdx.x; idx < sg.nrows * Q; idx += NW * kWave) {
    const int g = idx / Q;
    const int d = (idx % Q) * 4;
    const int h = sg.h0 + g;
    const int64_t row = ((int64_t)sg.b * a.heads + h) * ns + sid;
    *reinterpret_cast<f4_t*>(a.opart + row * D + d) = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
    if (d == 0) a.lse[((int64_t)sg.b * ns + sid) * a.heads + h] = kNegInf;
  }
}

// A thief's run: share, chunks [c0, c1), steal slot index (share < 0: none).
struct StealJob {
  int share, c0, c1, slot;
};

// One victim search and take by the whole workgroup (it synchronises; `job`
// is LDS for the broadcast). Returns share -1 when no share has an
// unclaimed chunk and a free steal slot, share -2 when the take lost a race
// (search again). Relaxed atomics suffice: the words pass no data, and the
// partials are read by the next launch.
template <int NW>
__device__ __forceinline__ StealJob steal_search(const SplitArgs& a, StealJob& job,
                                                 unsigned (&red)[NW]) {
  const int tid = threadIdx.x;
  // best key: unclaimed chunks (high bits), then the lowest share
  unsigned key = 0;
  for (int v = tid; v < a.steal_shares; v += NW * kWave) {
    const unsigned long long w =
        __hip_atomic_load(a.steal + v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int u = steal_unclaimed(w);
    if (steal_take(w, a.steal_cap).m > 0) {
      const unsigned k = ((unsigned)u << 12) | (unsigned)(kStealMaxShares - 1 - v);
      key = k > key ? k : key;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const unsigned o = __shfl_xor(key, off, kWave);
    key = o > key ? o : key;
  }
  if ((tid & (kWave - 1)) == 0) red[tid / kWave] = key;
  __syncthreads();
  if (tid == 0) {
    unsigned best = red[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) best = red[w] > best ? red[w] : best;
    StealJob j{-1, 0, 0, 0};
    if (best != 0) {
      const int v = kStealMaxShares - 1 - (int)(best & 4095u);
      unsigned long long* word = a.steal + v;
      unsigned long long w = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      j.share = -2;
      // the back half, rounded up: even a last unclaimed chunk is worth
      // taking (measured on MI355X, Llama B16/128K at 8 slots: taking only
      // from two or more unclaimed chunks, the floor half, 1240-1242 us;
      // this rule 1233-1235 us)
      const StealTake tk = steal_take(w, a.steal_cap);
      if (tk.m > 0 &&
          __hip_atomic_compare_exchange_strong(word, &w, tk.want, __ATOMIC_RELAXED,
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
        j = StealJob{v, tk.c0, tk.c1, tk.slot};
    }
    job = j;
  }
  __syncthreads();
  const StealJob j = job;
  __syncthreads();  // every thread has its copy before the next search writes
  return j;
}

// ------------------------------------------------------------ pipeline --
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
}

// A wave's walk over the tiles first, first+NW, ... (< nt) of a segment
// with PF tiles' loads in flight while it computes one: PF+1 register
// buffers used round-robin, the loop unrolled so every buffer index is a
// constant. The caller has already issued the load of tile `first` into
// buf[0]. Loads of tiles past the segment are harmless (empty descriptors
// return zeros without touching memory; skipping them costs registers);
// the walk stops after the last tile. The
// scheduling barriers keep each prefetch ahead of the compute it overlaps.
// hook(j) runs before each tile's step (before the load of tile j + PF*NW)
// and may extend nt.
template <int PF, int NW, typename Tile, typename Load, typename Compute, typename Hook>
__device__ __forceinline__ void tile_pipeline(int first, const int& nt, Tile (&buf)[PF + 1],
                                              Load&& load, Compute&& compute, Hook&& hook) {
  if (first >= nt) return;  // uniform: this wave has no tile of the segment
  static_for<PF - 1>([&](auto ui) {
    constexpr int u = decltype(ui)::value + 1;
    load(first + u * NW, buf[u]);
  });
  int j = first;
  while (true) {
    bool done = false;
    static_for<PF + 1>([&](auto ui) {
      constexpr int u = decltype(ui)::value;
      if (!done) {
        hook(j);
        load(j + PF * NW, buf[(u + PF) % (PF + 1)]);
        __builtin_amdgcn_sched_barrier(0);
        compute(j, buf[u]);
        __builtin_amdgcn_sched_barrier(0);
        j += NW;
        done = j >= nt;
      }
    });
    if (done) break;
  }
}

template <int PF, int NW, typename Tile, typename Load, typename Compute>
__device__ __forceinline__ void tile_pipeline(int first, const int& nt, Tile (&buf)[PF + 1],
                                              Load&& load, Compute&& compute) {
  tile_pipeline<PF, NW, Tile>(first, nt, buf, load, compute, [](int) {});
}

// --------------------------------------------------------- VALU kernel --
template <int DT, int D, int GC, bool NT, int NW, bool QUEUE>
__global__ __launch_bounds__(kWave* NW) void split_kernel(const int32_t* cu, int batch, SplitArgs a) {
  constexpr int EB = Elem<DT>::bytes;
  constexpr int EPL = 16 / EB;         // elements per 16-byte chunk
  constexpr int LPR = D / EPL;         // lanes per K/V row
  constexpr int RPI = kWave / LPR;     // rows per wave-wide load
  constexpr int NI = valu_loads_per_tile(EB, D);  // loads per tile (each of K and V)
  constexpr int TK = NI * RPI;         // keys per wave tile
  static_assert(LPR >= 1 && LPR <= 32 && (NI % 2) == 0, "unsupported geometry");

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  // wave index is uniform across the wave; say so, so tile bases and
  // buffer descriptors stay in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int rg = lane / LPR;  // which row of a load this lane holds
  const int c = lane % LPR;   // which 16-byte chunk of the row

  const SeqTable st{cu, batch};
  const LaneSeqs ls = lane_seqs(st);
  // q chunks of the packed rows of the current item (rows past the group
  // read as zero)
  u4_t q[GC];
  auto load_q = [&](const WorkItem& w, int b) {
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      if (g < w.nrows) {
        const char* qp = static_cast<const char*>(a.q) +
                         (((int64_t)b * a.heads + w.h0 + g) * D + c * EPL) * EB;
        q[g] = *reinterpret_cast<const u4_t*>(qp);
      } else {
        q[g] = u4_t{0u, 0u, 0u, 0u};
      }
    }
  };
  const float score_mul = DT == DT_F32 ? 1.0f : a.scale_log2;
  const uint32_t tsb = (uint32_t)(a.st * EB);
  const uint32_t lane_off = (uint32_t)rg * tsb + (uint32_t)c * 16u;

  // m: the lazily moved reference max of each lane group; mt: the true max
  float m[GC], mt[GC], l[GC], acc[GC][EPL];
  Segment sg;  // the current item's segment
  struct Tile {
    u4_t k[NI], v[NI];
  };
  auto load_tile_of = [&](const Segment& sgx, int j, Tile& t) {
    __amdgpu_buffer_rsrc_t rk, rv;
    tile_rsrc<TK, D * EB>(sgx, j, rk, rv);
#pragma unroll
    for (int i = 0; i < NI; ++i) t.k[i] = buffer_load16<NT>(rk, lane_off + (uint32_t)(i * RPI) * tsb);
#pragma unroll
    for (int i = 0; i < NI; ++i) t.v[i] = buffer_load16<NT>(rv, lane_off + (uint32_t)(i * RPI) * tsb);
  };
  auto load_tile = [&](int j, Tile& t) { load_tile_of(sg, j, t); };
  auto compute_tile = [&](int j, const Tile& t) {
    const u4_t(&kt)[NI] = t.k;
    const u4_t(&vt)[NI] = t.v;
    const int64_t nkeys = sg.nkeys;
    const int64_t k0 = (int64_t)j * TK;
    float s[NI][GC];
    bool valid[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      valid[i] = k0 + i * RPI + rg < nkeys;
#pragma unroll
      for (int g = 0; g < GC; ++g) {
        float part = group_sum<LPR>(chunk_dot<DT>(q[g], kt[i], 0.0f));
        s[i][g] = valid[i] ? part * score_mul : kNegInf;
      }
    }
    // lazy online-softmax rescale, per row of this lane group
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      float tmax = s[0][g];
#pragma unroll
      for (int i = 1; i < NI; ++i) tmax = fmaxf(tmax, s[i][g]);
      mt[g] = fmaxf(mt[g], tmax);
      if (tmax > m[g] + kLazyRescale) {
        const float alpha = fast_exp2(m[g] - tmax);
        l[g] *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] *= alpha;
        m[g] = tmax;
      }
    }
    float p[NI][GC];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int g = 0; g < GC; ++g) {
        p[i][g] = valid[i] ? fast_exp2(s[i][g] - m[g]) : 0.0f;
        l[g] += p[i][g];
      }
    // PV
    if constexpr (DT == DT_F32) {
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int g = 0; g < GC; ++g)
#pragma unroll
          for (int e = 0; e < EPL; ++e)
            acc[g][e] = __builtin_fmaf(p[i][g], __builtin_bit_cast(float, word(vt[i], e)), acc[g][e]);
    } else {
#pragma unroll
      for (int i = 0; i < NI; i += 2) {
        uint32_t pp[GC];
#pragma unroll
        for (int g = 0; g < GC; ++g) pp[g] = pack_pair<DT>(p[i][g], p[i + 1][g]);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          // (v_i[2w], v_{i+1}[2w]) and (v_i[2w+1], v_{i+1}[2w+1])
          const uint32_t lo = __builtin_amdgcn_perm(word(vt[i + 1], w), word(vt[i], w), 0x05040100u);
          const uint32_t hi = __builtin_amdgcn_perm(word(vt[i + 1], w), word(vt[i], w), 0x07060302u);
#pragma unroll
          for (int g = 0; g < GC; ++g) {
            acc[g][2 * w] = pair_dot<DT>(pp[g], lo, acc[g][2 * w]);
            acc[g][2 * w + 1] = pair_dot<DT>(pp[g], hi, acc[g][2 * w + 1]);
          }
        }
      }
    }
  };

  Tile buf[kPrefetchTilesValu + 1];
  __shared__ int sm_next;
  int item = blockIdx.x;
  while (true) {
    const WorkItem wi = decode_item<GC>(a, item);
    load_q(wi, wi.rank);  // guess: sequence == rank (equal lengths)
    sg = locate_segment<EB>(a, st, wi, ls);
    if (sg.b != wi.rank) load_q(wi, sg.b);
    load_tile_of(sg, wave, buf[0]);
    if constexpr (DT == DT_F32) {
#pragma unroll
      for (int g = 0; g < GC; ++g)
#pragma unroll
        for (int w = 0; w < 4; ++w)
          q[g][w] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, word(q[g], w)) * a.scale_log2);
    }
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      m[g] = kNegInf;
      mt[g] = kNegInf;
      l[g] = 0.0f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] = 0.0f;
    }
    const int nt = (int)((sg.nkeys + TK - 1) / TK);
    tile_pipeline<kPrefetchTilesValu, NW, Tile>(wave, nt, buf, load_tile, compute_tile);

    // ---- merge the lane groups of this wave onto the wave's true max ----
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      const float M = across_groups<LPR>(mt[g], OpMax{});
      const float f = m[g] == kNegInf ? 0.0f : fast_exp2(m[g] - M);
      l[g] = across_groups<LPR>(l[g] * f, OpAdd{});
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] = across_groups<LPR>(acc[g][e] * f, OpAdd{});
      m[g] = M;
    }

    // ---- merge the waves through LDS and write the epilogue ----
    __shared__ float sm_m[NW][GC];
    __shared__ float sm_l[NW][GC];
    __shared__ __attribute__((aligned(16))) float sm_acc[NW][GC][D];
    if (rg == 0) {
#pragma unroll
      for (int g = 0; g < GC; ++g) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) sm_acc[wave][g][c * EPL + e] = acc[g][e];
        if (c == 0) {
          sm_m[wave][g] = m[g];
          sm_l[wave][g] = l[g];
        }
      }
    }
    __syncthreads();
    store_segment<DT, D, GC, NW>(a, sg, sm_m, sm_l, sm_acc);
    if constexpr (!QUEUE) {  // static schedule: the loop body runs once
      if (a.arrivals != nullptr) arrive_and_merge<DT, D, NW>(a, sg, item / a.num_splits, sm_next);
      break;
    }
    item = claim_next(a, sm_next);
    if (item >= a.items) break;
  }
}

// --------------------------------------------------------- MFMA kernel --
// Same contract as split_kernel, at head dim 128, with QK^T on the matrix
// cores. Per wave tile of 16 keys, for fp16/bf16:
//  * S^T[16 keys x 16 cols] = K[16 x 128] . Q^T[128 x 16] as four
//    v_mfma_f32_16x16x32_{f16,bf16}: lane (R = lane/16, c = lane%16) feeds
//    row c of K (dims 32m + 8R .. +8 for step m, one 16-byte load each) and
//    column c of Q^T (query row c of the group, zero past the group), and
//    receives S for query row g = c and keys 4R + r, r = 0..3.
//  * Online softmax runs per lane on those four scores (per (R, g) running
//    max and sum, lazily rescaled as in split_kernel): no cross-lane work.
//  * PV stays on the VALU with v_dot2: lane (R, c) holds dims 8c..8c+7 of
//    keys 4R + i (V loads of whole 256-byte rows) and takes the packed
//    probability pair of query row g from lane (R, g) of its own 16-lane row
//    with DPP row_newbcast.
// For fp32 (v_mfma_f32_16x16x4_f32, full fp32 products and sums):
//  * S^T = K . Q^T in 32 steps of 4 dims: lane (R, c) loads 16-byte chunks
//    R, R + 4, ..., R + 28 of K row c and of query row c, and step (i, e)
//    takes element e of chunk R + 4i (lane group R supplies k index R of
//    each step); the scores land as above (query row c, keys 4R..4R+3).
//  * PV with fp32 FMAs: lane (R, c) holds dims 4c..4c+3 and 64+4c..64+4c+3
//    of keys 4R + i (chunks c and c + 16: whole rows per load) and takes each
//    probability of query row g from lane (R, g) with row_newbcast.
// The workgroup epilogue is shared with split_kernel.
template <int LANE>
__device__ __forceinline__ uint32_t row_bcast(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x150 + LANE, 0xF, 0xF, false);
}

template <int LANE>
__device__ __forceinline__ float row_bcast(float x) {
  return __builtin_bit_cast(float, row_bcast<LANE>(__builtin_bit_cast(uint32_t, x)));
}

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef __bf16 b8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f4_t mfma_qk_f32(float k, float q, f4_t acc) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(k, q, acc, 0, 0, 0);
}

template <int DT>
__device__ __forceinline__ f4_t mfma_qk(const u4_t& k, const u4_t& q, f4_t acc) {
  if constexpr (DT == DT_F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, k),
                                                  __builtin_bit_cast(h8_t, q), acc, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8_t, k),
                                                   __builtin_bit_cast(b8_t, q), acc, 0, 0, 0);
}

template <int DT, int GC, bool NT, int SCH>
__global__ __launch_bounds__(kWave* kWavesMfma) void split_kernel_mfma(const int32_t* cu, int batch, SplitArgs a) {
  static_assert(GC <= 16, "one 16-column MFMA tile of query rows");
  constexpr bool F32 = DT == DT_F32;
  constexpr int D = 128;
  constexpr int EB = Elem<DT>::bytes;
  constexpr int TK = 16;           // keys per wave tile
  constexpr int KS = F32 ? 8 : D / 32;  // 16-byte K (and Q) chunks per lane per tile
  constexpr int VL = F32 ? 8 : 4;       // 16-byte V chunks per lane per tile
  constexpr int NW = kWavesMfma;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int R = lane >> 4;   // key group of this lane
  const int c = lane & 15;   // K row / query row / V chunk of this lane

  const SeqTable st{cu, batch};
  const LaneSeqs ls = lane_seqs(st);
  // Q^T as the MFMA B operand: column c = query row h0 + c of the current
  // item (zero past the group)
  u4_t qb[KS];
  auto load_q = [&](const WorkItem& w, int b) {
#pragma unroll
    for (int m = 0; m < KS; ++m) {
      if (c < w.nrows) {
        // fp16/bf16: dims 32m + 8R..+8; fp32: chunk R + 4m (dims 16m + 4R..+4)
        const int d0 = F32 ? 16 * m + 4 * R : 32 * m + 8 * R;
        const char* qp = static_cast<const char*>(a.q) +
                         (((int64_t)b * a.heads + w.h0 + c) * D + d0) * EB;
        qb[m] = *reinterpret_cast<const u4_t*>(qp);
      } else {
        qb[m] = u4_t{0u, 0u, 0u, 0u};
      }
    }
  };
  const uint32_t tsb = (uint32_t)(a.st * EB);
  // fp16/bf16: K and V are both loaded as whole rows: lane (R, c) gets
  // 16-byte chunk c of rows 4R + i, i = 0..3 (one wave-wide load = 4 full
  // 256-byte rows). fp32: V likewise (chunks c and c + 16 of rows 4R + i),
  // K in the matrix-core layout (chunks R + 4i of row c).
  const uint32_t kv_off = (uint32_t)(4 * R) * tsb + (uint32_t)c * 16u;  // + i*tsb
  const uint32_t k32_off = (uint32_t)c * tsb + (uint32_t)R * 16u;       // + 64*i
  // fp16/bf16 K is regrouped through LDS into the matrix-core layout: row
  // stride 17 chunks (272 bytes) keeps both the writes and the reads free
  // of bank conflicts.
  constexpr int kLdsRow = 17;
  __shared__ u4_t lds_k[F32 ? 1 : NW][16 * kLdsRow];
  u4_t* const my_k = lds_k[F32 ? 0 : wave];

  // for (key group R, query row c): the lazily moved reference max, the
  // true max, and the sum relative to the reference
  float m_run, m_true, l_run;
  float acc[GC][8];
  Segment sg;  // the current item's segment
  struct Tile {
    u4_t k[KS], v[VL];
  };
  auto load_tile_of = [&](const Segment& sgx, int j, Tile& t) {
    __amdgpu_buffer_rsrc_t rk, rv;
    tile_rsrc<TK, D * EB>(sgx, j, rk, rv);
    if constexpr (F32) {
#pragma unroll
      for (int i = 0; i < KS; ++i) t.k[i] = buffer_load16<NT>(rk, k32_off + (uint32_t)i * 64u);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          t.v[2 * i + h] = buffer_load16<NT>(rv, kv_off + (uint32_t)i * tsb + (uint32_t)h * 256u);
    } else {
#pragma unroll
      for (int i = 0; i < KS; ++i) t.k[i] = buffer_load16<NT>(rk, kv_off + (uint32_t)i * tsb);
#pragma unroll
      for (int i = 0; i < 4; ++i) t.v[i] = buffer_load16<NT>(rv, kv_off + (uint32_t)i * tsb);
    }
  };
  auto load_tile = [&](int j, Tile& t) { load_tile_of(sg, j, t); };

  auto compute_tile = [&](int j, const Tile& t) {
    const u4_t(&vt)[VL] = t.v;
    const int64_t nkeys = sg.nkeys;
    f4_t s4 = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (F32) {
      // step (i, e): element e of chunk R + 4i, of K row c and query row c.
      // Four accumulators of eight steps each, added pairwise: the sum's
      // rounding error grows with the length of the sequential chain
      // (32 steps in one accumulator cost 2x the fp32 tolerance at 23x
      // the default scale; this keeps the depth near the VALU kernel's tree).
      f4_t sa[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) sa[e] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int i = 0; i < KS; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sa[e] = mfma_qk_f32(__builtin_bit_cast(float, word(t.k[i], e)),
                              __builtin_bit_cast(float, word(qb[i], e)), sa[e]);
      s4 = (sa[0] + sa[1]) + (sa[2] + sa[3]);
    } else {
      // K rows 4R + i, chunk c -> LDS -> lane (R, c) takes chunk 4m + R of
      // row c for MFMA step m (the k order is the same for Q, see load_q).
      // One wave writes and reads its own slice; LDS instructions of a wave
      // complete in order, so no barrier is needed.
#pragma unroll
      for (int i = 0; i < KS; ++i) my_k[(4 * R + i) * kLdsRow + c] = t.k[i];
      u4_t kt[KS];
#pragma unroll
      for (int m = 0; m < KS; ++m) kt[m] = my_k[c * kLdsRow + 4 * m + R];
#pragma unroll
      for (int m = 0; m < KS; ++m) s4 = mfma_qk<DT>(kt[m], qb[m], s4);
    }
    const int64_t kbase = (int64_t)j * TK + 4 * R;
    float s[4];
    bool valid[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      valid[r] = kbase + r < nkeys;
      s[r] = valid[r] ? s4[r] * a.scale_log2 : kNegInf;
    }
    const float tmax = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    m_true = fmaxf(m_true, tmax);
    const bool need = tmax > m_run + kLazyRescale;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {  // uniform, rare after the first tile
      float alpha = 1.0f;
      if (need) {
        alpha = fast_exp2(m_run - tmax);
        l_run *= alpha;
        m_run = tmax;
      }
      static_for<GC>([&](auto gi) {
        constexpr int g = decltype(gi)::value;
        const float ag = row_bcast<g>(alpha);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] *= ag;
      });
    }
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = valid[r] ? fast_exp2(s[r] - m_run) : 0.0f;
      l_run += p[r];
    }
    if constexpr (F32) {
      // acc[g][4h + e] += p(key 4R + i, row g) * V[key 4R + i][64h + 4c + e]
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        static_for<GC>([&](auto gi) {
          constexpr int g = decltype(gi)::value;
          const float pg = row_bcast<g>(p[i]);
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc[g][4 * h + e] = __builtin_fmaf(
                  pg, __builtin_bit_cast(float, word(vt[2 * i + h], e)), acc[g][4 * h + e]);
        });
      }
      return;
    } else {
    const uint32_t P[2] = {pack_pair<DT>(p[0], p[1]), pack_pair<DT>(p[2], p[3])};
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      uint32_t lo[4], hi[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        lo[w] = __builtin_amdgcn_perm(word(vt[2 * pr + 1], w), word(vt[2 * pr], w), 0x05040100u);
        hi[w] = __builtin_amdgcn_perm(word(vt[2 * pr + 1], w), word(vt[2 * pr], w), 0x07060302u);
      }
      static_for<GC>([&](auto gi) {
        constexpr int g = decltype(gi)::value;
        const uint32_t pp = row_bcast<g>(P[pr]);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          acc[g][2 * w] = pair_dot<DT>(pp, lo[w], acc[g][2 * w]);
          acc[g][2 * w + 1] = pair_dot<DT>(pp, hi[w], acc[g][2 * w + 1]);
        }
      });
    }
    }
  };

  Tile buf[kPrefetchTilesMfma + 1];
  __shared__ int sm_next;
  int item = blockIdx.x;
  // steal schedule: the current run, first the owner's of share blockIdx.x
  StealJob job{(int)blockIdx.x, 0, 1, 0};
  bool owner = true;
  [[maybe_unused]] int searches = 0;
  __shared__ int sm_claim[2];
  __shared__ int sm_steals;
  __shared__ StealJob sm_job;
  __shared__ unsigned sm_red[NW];
  while (true) {
    if constexpr (SCH == kSchedSteal) {
      const int unit = job.share / a.steal_nsh, r = job.share % a.steal_nsh;
      item = unit * a.num_splits + r * (1 + a.steal_cap) + (owner ? 0 : 1 + job.slot);
    }
    const WorkItem wi = decode_item<GC>(a, item);
    load_q(wi, wi.rank);  // guess: sequence == rank (equal lengths)
    [[maybe_unused]] Share sh{};
    if constexpr (SCH == kSchedSteal) {
      int b, cu0, cu1;
      sequence_of(st, wi, ls, b, cu0, cu1);
      const int64_t L = cu1 > cu0 ? (int64_t)cu1 - cu0 : 0;
      sh = share_of(L, job.share % a.steal_nsh, a.steal_nsh, a.steal_chunks);
      sg = segment_at<EB>(a, wi, b, cu0, sh.start + (int64_t)job.c0 * sh.ck,
                          sh.start + min((int64_t)job.c1 * sh.ck, sh.len));
    } else {
      sg = locate_segment<EB>(a, st, wi, ls);
    }
    if (sg.b != wi.rank) load_q(wi, sg.b);
    load_tile_of(sg, wave, buf[0]);
    m_run = kNegInf;
    m_true = kNegInf;
    l_run = 0.0f;
#pragma unroll
    for (int g = 0; g < GC; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] = 0.0f;
    int nt = (int)((sg.nkeys + TK - 1) / TK);
    if constexpr (SCH == kSchedSteal) {
      // The owner's run grows a chunk at a time. Thread 0 claims chunk
      // `owned` a chunk ahead; at the step before any wave would load a tile
      // of that chunk (every wave has tpw steps per full chunk), it
      // publishes the result, and the workgroup extends the run or ends it.
      // The barrier sits at the same step of every wave, and every chunk
      // before the last one is full, so every wave reaches it.
      unsigned long long pending = 0;  // thread 0: word value its claim returns
      int parity = 0;
      const int tpw = (int)(sh.ck / (TK * NW));
      int hook_step = owner && sh.nc >= 2 ? tpw - kPrefetchTilesMfma : INT_MAX;
      unsigned long long* const word = a.steal + job.share;
      if (owner && tid == 0) {
        sm_steals = 0;
        if (sh.nc >= 2)  // claims chunk 1 and publishes the chunk count
          pending = __hip_atomic_fetch_add(word, steal_first_claim(sh.nc), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
      }
      auto grow = [&](int j) {
        if ((j - wave) / NW != hook_step) return;  // uniform
        if (tid == 0) {
          const int chunk = steal_claimed_chunk(pending, sh.nc);
          sm_steals = steal_count(pending);  // final once the claims end
          sm_claim[parity] = chunk;
          if (chunk >= 0 && chunk + 1 < sh.nc)
            pending = __hip_atomic_fetch_add(word, kStealClaim, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        const int got = sm_claim[parity];  // two slots: the next write is two barriers away
        parity ^= 1;
        if (got >= 0) {
          const int owned = got + 1;
          sg.nkeys = min((int64_t)owned * sh.ck, sh.len);
          nt = (int)((sg.nkeys + TK - 1) / TK);
          hook_step = owned < sh.nc ? hook_step + tpw : INT_MAX;
        } else {
          hook_step = INT_MAX;
        }
      };
      tile_pipeline<kPrefetchTilesMfma, NW, Tile>(wave, nt, buf, load_tile, compute_tile, grow);
    } else {
      tile_pipeline<kPrefetchTilesMfma, NW, Tile>(wave, nt, buf, load_tile, compute_tile);
    }

    // ---- merge the four key groups R of this wave onto its true max ----
    const float M = across_groups<16>(m_true, OpMax{});
    const float f = m_run == kNegInf ? 0.0f : fast_exp2(m_run - M);
    const float lw = across_groups<16>(l_run * f, OpAdd{});
    // value v = 8g + e (query row g, element e of this lane: dim 8c + e, or
    // for fp32 dim 64 (e / 4) + 4c + e % 4), scaled onto M, then summed over
    // the four rows R by a reduce-scatter: lane (R, c) ends with the wave's
    // total of value 4j + R, i.e. row g = j / 2, element 4 (j % 2) + R.
    constexpr int NV = GC * 8;
    float x[NV];
    static_for<GC>([&](auto gi) {
      constexpr int g = decltype(gi)::value;
      const float fg = row_bcast<g>(f);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[8 * g + e] = acc[g][e] * fg;
    });
    float s2[NV / 2];
#pragma unroll
    for (int i = 0; i < NV / 2; ++i) s2[i] = rows_scatter(x[2 * i], x[2 * i + 1]);
    float s4[NV / 4];
#pragma unroll
    for (int j = 0; j < NV / 4; ++j) s4[j] = halves_scatter(s2[2 * j], s2[2 * j + 1]);

    // ---- merge the waves through LDS and write the epilogue ----
    __shared__ float sm_m[NW][GC];
    __shared__ float sm_l[NW][GC];
    __shared__ __attribute__((aligned(16))) float sm_acc[NW][GC][D];
#pragma unroll
    for (int j = 0; j < NV / 4; ++j)
      sm_acc[wave][j / 2][F32 ? 64 * (j % 2) + 4 * c + R : 8 * c + 4 * (j % 2) + R] = s4[j];
    if (R == 0 && c < GC) {
      sm_m[wave][c] = M;
      sm_l[wave][c] = lw;
    }
    __syncthreads();
    store_segment<DT, D, GC, NW>(a, sg, sm_m, sm_l, sm_acc);
    if constexpr (SCH == kSchedStatic) {  // the loop body runs once
      if (a.arrivals != nullptr) arrive_and_merge<DT, D, NW>(a, sg, item / a.num_splits, sm_next);
      break;
    } else if constexpr (SCH == kSchedQueue) {
      item = claim_next(a, sm_next);
      if (item >= a.items) break;
    } else {
      if (owner) {  // steal slots no thief took: empty partials
        const int taken = sm_steals;
        for (int s = 1 + taken; s <= a.steal_cap; ++s) store_empty<D, NW>(a, sg, sg.sid + s);
        owner = false;
      }
      StealJob j;
      do {
        j = steal_search<NW>(a, sm_job, sm_red);
      } while (j.share == -2 && ++searches < kStealScans);
      if (j.share < 0 || ++searches > kStealScans) break;
      job = j;
    }
  }
}


// Dynamic LDS that, added to the kernel's static LDS, lets exactly
// kMfmaWorkgroupsPerCu matrix-core workgroups reside on one compute unit
// (0 if the device's per-workgroup limit does not allow it). Computed once
// per kernel instance.
template <int DT, int GC, bool NT, int SCH>
size_t mfma_lds_reserve() {
  static const size_t bytes = [] {
    hipFuncAttributes fa;
    if (hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(
                                      &split_kernel_mfma<DT, GC, NT, SCH>)) != hipSuccess) {
      (void)hipGetLastError();
      return (size_t)0;
    }
    int dev = 0, max_block = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&max_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
            hipSuccess) {
      (void)hipGetLastError();
      return (size_t)0;
    }
    // per-workgroup total just under kLdsBytesPerCu / k: k fit, k + 1 do not
    const long total = (long)kLdsBytesPerCu / kMfmaWorkgroupsPerCu - 1024;
    const long dyn = total - (long)fa.sharedSizeBytes;
    if (dyn <= 0 || total > (long)max_block) return (size_t)0;
    return (size_t)dyn;
  }();
  return bytes;
}

#ifndef FD_QUEUE_PER_CU
#define FD_QUEUE_PER_CU 1
#endif
// Workgroups per compute unit of a queue-scheduled launch (0: as many as
// fit, i.e. the kernel's occupancy). Measured on MI355X (varlen Qwen batch,
// 8 splits, 1024 segments): one per compute unit 184.7 us, two (the
// matrix-core kernel's occupancy) 198.2 us, static schedule 195.1 us: a
// second resident workgroup doubles the bytes in flight per compute unit,
// which streams slower, as in the static launches.
constexpr int kQueueWorkgroupsPerCu = FD_QUEUE_PER_CU;

// Grid of a queue-scheduled launch: kQueueWorkgroupsPerCu (at most this
// kernel's occupancy) workgroups per compute unit, never more than the
// segments. Computed once per kernel instance.
template <typename Tag>
dim3 queue_grid(const SplitArgs& a, const void* kernel, int block, size_t lds) {
  static const int per_cu = [&] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, block, lds) != hipSuccess ||
        n < 1) {
      (void)hipGetLastError();
      n = 1;
    }
    return kQueueWorkgroupsPerCu > 0 && kQueueWorkgroupsPerCu < n ? kQueueWorkgroupsPerCu : n;
  }();
  const long g = (long)per_cu * (a.cus > 0 ? a.cus : 1);
  return dim3((unsigned)(g < (long)a.items ? g : (long)a.items));
}

template <int DT, int GC, bool NT, int SCH>
struct MfmaTag {};
template <int DT, int D, int GC, bool NT, int NW, bool QUEUE>
struct ValuTag {};

template <int DT, int GC, bool NT, int SCH>
hipError_t launch_mfma(const SplitArgs& a, dim3 grid, hipStream_t s) {
  const dim3 block(kWave * kWavesMfma);
  const size_t lds = mfma_lds_reserve<DT, GC, NT, SCH>();
  if constexpr (SCH == kSchedQueue)
    grid = queue_grid<MfmaTag<DT, GC, NT, SCH>>(
        a, reinterpret_cast<const void*>(&split_kernel_mfma<DT, GC, NT, SCH>), block.x, lds);
  hipLaunchKernelGGL((split_kernel_mfma<DT, GC, NT, SCH>), grid, block, lds, s, a.cu, a.batch,
                     a);
  return hipGetLastError();
}

template <int DT, int D, int GC, bool NT, int NW, bool QUEUE>
hipError_t launch_valu(const SplitArgs& a, dim3 grid, hipStream_t s) {
  const dim3 block(kWave * NW);
  if constexpr (QUEUE)
    grid = queue_grid<ValuTag<DT, D, GC, NT, NW, QUEUE>>(
        a, reinterpret_cast<const void*>(&split_kernel<DT, D, GC, NT, NW, QUEUE>), block.x, 0);
  hipLaunchKernelGGL((split_kernel<DT, D, GC, NT, NW, QUEUE>), grid, block, 0, s, a.cu, a.batch,
                     a);
  return hipGetLastError();
}

// f(std::integral_constant<int, rows>) for rows in 1..kMaxRowsPerPass.
template <typename F>
hipError_t by_rows(int rows, F&& f) {
  switch (rows) {
    case 1: return f(std::integral_constant<int, 1>{});
    case 2: return f(std::integral_constant<int, 2>{});
    case 3: return f(std::integral_constant<int, 3>{});
    case 4: return f(std::integral_constant<int, 4>{});
    case 5: return f(std::integral_constant<int, 5>{});
    case 6: return f(std::integral_constant<int, 6>{});
    case 7: return f(std::integral_constant<int, 7>{});
    case 8: return f(std::integral_constant<int, 8>{});
    default: return hipErrorInvalidValue;
  }
}

// Host-side dispatch over (path, D, rows) for one dtype. The matrix-core
// kernel exists at head dim 128; VALU launches below one pass
// (never non-temporal, never queued) take 8-wave VALU workgroups.
template <int DT, int D, bool NT, bool QUEUE>
hipError_t launch_split_dnq(const SplitArgs& a, int rows, bool mfma, dim3 grid, hipStream_t s) {
  if constexpr (D == 128) {
    if (mfma)
      return by_rows(rows, [&](auto r) {
        return launch_mfma<DT, decltype(r)::value, NT, QUEUE ? kSchedQueue : kSchedStatic>(
            a, grid, s);
      });
  }
  if constexpr (!NT && !QUEUE) {
    if (a.wide)
      return by_rows(rows, [&](auto r) {
        return launch_valu<DT, D, decltype(r)::value, NT, kWavesValuWide, QUEUE>(a, grid, s);
      });
  }
  return by_rows(rows, [&](auto r) {
    return launch_valu<DT, D, decltype(r)::value, NT, kWavesValu, QUEUE>(a, grid, s);
  });
}

// The queue schedule is only taken by launches that fill the device (which
// always carry non-temporal K/V loads); the host never asks for it elsewhere.
// The steal schedule exists in the matrix-core kernel; the host asks for it
// only there (grid: one workgroup per share).
template <int DT, int D>
hipError_t launch_split_d(const SplitArgs& a, int rows, bool mfma, dim3 grid, hipStream_t s) {
  if (a.steal != nullptr) {
    if constexpr (D == 128) {
      if (mfma)
        return by_rows(rows, [&](auto r) {
          return launch_mfma<DT, decltype(r)::value, true, kSchedSteal>(a, grid, s);
        });
    }
    return hipErrorInvalidValue;
  }
  if (a.queue != nullptr && a.kv_nt)
    return launch_split_dnq<DT, D, true, true>(a, rows, mfma, grid, s);
  return a.kv_nt ? launch_split_dnq<DT, D, true, false>(a, rows, mfma, grid, s)
                 : launch_split_dnq<DT, D, false, false>(a, rows, mfma, grid, s);
}

template <int DT>
hipError_t launch_split_dt(const SplitArgs& a, int dim, int rows, bool mfma, dim3 grid,
                           hipStream_t s) {
  switch (dim) {
    case 16: return launch_split_d<DT, 16>(a, rows, mfma, grid, s);
    case 32: return launch_split_d<DT, 32>(a, rows, mfma, grid, s);
    case 64: return launch_split_d<DT, 64>(a, rows, mfma, grid, s);
    case 128: return launch_split_d<DT, 128>(a, rows, mfma, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fd
