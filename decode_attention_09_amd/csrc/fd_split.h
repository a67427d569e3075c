// Split kernel of flash decoding for gfx950: one workgroup per
// (split, KV head, row chunk, sequence) computes, for the packed query rows
// of one GQA group, the online-softmax partial output of its KV segment and
// the segment's base-2 log-sum-exp.
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
//    than 2^8, so rescaling is rare and p stays <= 256.
//  * PV: p for two keys is packed to fp16x2/bf16x2 and multiplied with the
//    matching pair of V elements (v_perm regroups them) by v_dot2, fp32 acc.
//  * Bounds: each tile's K/V loads go through a buffer descriptor whose
//    size ends at the last valid row of the segment, so rows past the
//    segment (or the tensor) read as zero without branches, and are then
//    masked out of the softmax.
//  * Four waves per workgroup take interleaved tiles of the segment and are
//    merged through LDS at the end (the same LSE merge as the combine).
//  * Double-buffered register tiles: the next tile's loads are issued
//    before the current tile is computed.
#pragma once

#include "fd_internal.h"

namespace fd {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

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

// Sum over aligned groups of LPR lanes; every lane of a group gets the same
// (bitwise) result because each butterfly step adds the same two values.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (LPR >= 2) x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
  if constexpr (LPR >= 4) x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
  if constexpr (LPR >= 8) x += dpp_mov<0x141>(x);  // row_half_mirror
  if constexpr (LPR >= 16) x += dpp_mov<0x140>(x); // row_mirror
  if constexpr (LPR >= 32) x += __shfl_xor(x, 16);
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

__device__ __forceinline__ u4_t buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0));
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

// --------------------------------------------------------------- kernel --
template <int DT, int D, int GC>
__global__ __launch_bounds__(kWave* kWavesPerGroup) void split_kernel(SplitArgs a) {
  constexpr int EB = Elem<DT>::bytes;
  constexpr int EPL = 16 / EB;         // elements per 16-byte chunk
  constexpr int LPR = D / EPL;         // lanes per K/V row
  constexpr int RPI = kWave / LPR;     // rows per wave-wide load
  constexpr int NI = kLoadsPerTile;    // loads per tile (each of K and V)
  constexpr int TK = NI * RPI;         // keys per wave tile
  constexpr int NW = kWavesPerGroup;
  static_assert(LPR >= 1 && LPR <= 32 && (NI % 2) == 0, "unsupported geometry");

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  // wave index is uniform across the wave; say so, so tile bases and
  // buffer descriptors stay in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int rg = lane / LPR;  // which row of a load this lane holds
  const int c = lane % LPR;   // which 16-byte chunk of the row

  // workgroup -> (split, KV head, row chunk, sequence); split fastest.
  int wg = blockIdx.x;
  const int ns = a.num_splits;
  const int sid = wg % ns;
  wg /= ns;
  const int hcn = a.kv_heads * a.row_chunks;
  const int hc = wg % hcn;
  const int b = wg / hcn;
  const int kvh = hc / a.row_chunks;
  const int chunk = hc % a.row_chunks;
  const int h0 = kvh * a.group + chunk * kMaxRowsPerPass;
  const int nrows = min(GC, a.group - chunk * kMaxRowsPerPass);

  // varlen bounds and proportional segment (64-bit products)
  const int cu0 = a.cu[b];
  const int cu1 = a.cu[b + 1];
  const int64_t L = cu1 > cu0 ? (int64_t)cu1 - cu0 : 0;
  const int64_t seg0 = L * sid / ns;
  const int64_t nkeys = L * (sid + 1) / ns - seg0;

  // q chunks of the packed rows (rows past the group read as zero)
  u4_t q[GC];
#pragma unroll
  for (int g = 0; g < GC; ++g) {
    if (g < nrows) {
      const char* qp = static_cast<const char*>(a.q) +
                       (((int64_t)b * a.heads + h0 + g) * D + c * EPL) * EB;
      q[g] = *reinterpret_cast<const u4_t*>(qp);
    } else {
      q[g] = u4_t{0u, 0u, 0u, 0u};
    }
    if constexpr (DT == DT_F32) {
#pragma unroll
      for (int w = 0; w < 4; ++w)
        q[g][w] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, word(q[g], w)) * a.scale_log2);
    }
  }
  const float score_mul = DT == DT_F32 ? 1.0f : a.scale_log2;

  const int64_t row0 = (int64_t)b * a.sb + (int64_t)cu0 * a.scu + (int64_t)kvh * a.sh + seg0 * a.st;
  const char* kseg = static_cast<const char*>(a.k) + row0 * EB;
  const char* vseg = static_cast<const char*>(a.v) + row0 * EB;
  const uint32_t tsb = (uint32_t)(a.st * EB);  // bytes between consecutive keys
  const uint32_t lane_off = (uint32_t)rg * tsb + (uint32_t)c * 16u;

  float m[GC], l[GC], acc[GC][EPL];
#pragma unroll
  for (int g = 0; g < GC; ++g) {
    m[g] = kNegInf;
    l[g] = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.0f;
  }

  const int nt = (int)((nkeys + TK - 1) / TK);

  // Loads of tile j; a tile past the segment gets an empty descriptor, so
  // the loads are unconditional and return zeros.
  auto load_tile = [&](int j, u4_t (&kt)[NI], u4_t (&vt)[NI]) {
    const int64_t k0 = (int64_t)j * TK;
    const int64_t nv = nkeys - k0;
    const uint32_t rec = nv > 0 ? (uint32_t)((min(nv, (int64_t)TK) - 1) * tsb + D * EB) : 0u;
    const char* kb = kseg + (nv > 0 ? k0 * tsb : 0);
    const char* vb = vseg + (nv > 0 ? k0 * tsb : 0);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb, rec);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb, rec);
#pragma unroll
    for (int i = 0; i < NI; ++i) kt[i] = buffer_load16(rk, lane_off + (uint32_t)(i * RPI) * tsb);
#pragma unroll
    for (int i = 0; i < NI; ++i) vt[i] = buffer_load16(rv, lane_off + (uint32_t)(i * RPI) * tsb);
  };

  auto compute_tile = [&](int j, const u4_t (&kt)[NI], const u4_t (&vt)[NI]) {
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

  {
    u4_t ka[NI], va[NI], kb[NI], vb[NI];
    int j = wave;
    load_tile(j, ka, va);
    // The scheduling barriers keep each prefetch ahead of the compute it
    // overlaps (the scheduler would otherwise sink loads past waits).
    while (j < nt) {
      load_tile(j + NW, kb, vb);
      __builtin_amdgcn_sched_barrier(0);
      compute_tile(j, ka, va);
      __builtin_amdgcn_sched_barrier(0);
      j += NW;
      if (j >= nt) break;
      load_tile(j + NW, ka, va);
      __builtin_amdgcn_sched_barrier(0);
      compute_tile(j, kb, vb);
      __builtin_amdgcn_sched_barrier(0);
      j += NW;
    }
  }

  // ---- merge the lane groups of this wave (each has its own max) ----
#pragma unroll
  for (int g = 0; g < GC; ++g) {
    float M = m[g];
#pragma unroll
    for (int mask = LPR; mask < kWave; mask <<= 1) M = fmaxf(M, __shfl_xor(M, mask));
    const float f = m[g] == kNegInf ? 0.0f : fast_exp2(m[g] - M);
    l[g] *= f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] *= f;
#pragma unroll
    for (int mask = LPR; mask < kWave; mask <<= 1) {
      l[g] += __shfl_xor(l[g], mask);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] += __shfl_xor(acc[g][e], mask);
    }
    m[g] = M;
  }

  // ---- merge the waves through LDS and write the epilogue ----
  __shared__ float sm_m[NW][GC];
  __shared__ float sm_l[NW][GC];
  __shared__ float sm_acc[NW][GC][D];
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

  for (int idx = tid; idx < nrows * D; idx += NW * kWave) {
    const int g = idx / D;
    const int d = idx % D;
    float M = sm_m[0][g];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, sm_m[w][g]);
    float lsum = 0.0f, o = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = sm_m[w][g] == kNegInf ? 0.0f : fast_exp2(sm_m[w][g] - M);
      lsum += f * sm_l[w][g];
      o += f * sm_acc[w][g][d];
    }
    const bool any = lsum > 0.0f;
    o = any ? o / lsum : 0.0f;
    const int h = h0 + g;
    if (a.direct) {
      store_out<DT>(a.out, ((int64_t)b * a.heads + h) * D + d, o);
    } else {
      a.opart[(((int64_t)b * a.heads + h) * ns + sid) * D + d] = o;
      if (d == 0)
        a.lse[((int64_t)b * ns + sid) * a.heads + h] = any ? fast_log2(lsum) + M : kNegInf;
    }
  }
}

// Host-side dispatch over (D, rows) for one dtype.
template <int DT, int D>
hipError_t launch_split_d(const SplitArgs& a, int rows, dim3 grid, hipStream_t s) {
  dim3 block(kWave * kWavesPerGroup);
  switch (rows) {
#define FD_CASE(R) \
  case R: hipLaunchKernelGGL((split_kernel<DT, D, R>), grid, block, 0, s, a); break;
    FD_CASE(1) FD_CASE(2) FD_CASE(3) FD_CASE(4) FD_CASE(5) FD_CASE(6) FD_CASE(7) FD_CASE(8)
#undef FD_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int DT>
hipError_t launch_split_dt(const SplitArgs& a, int dim, int rows, dim3 grid, hipStream_t s) {
  switch (dim) {
    case 16: return launch_split_d<DT, 16>(a, rows, grid, s);
    case 32: return launch_split_d<DT, 32>(a, rows, grid, s);
    case 64: return launch_split_d<DT, 64>(a, rows, grid, s);
    case 128: return launch_split_d<DT, 128>(a, rows, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fd
