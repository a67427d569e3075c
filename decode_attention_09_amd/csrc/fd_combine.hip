// Combine kernel of flash decoding for gfx950: merges the per-split
// normalised partial outputs with their base-2 log-sum-exps,
//
//   M = max_s lse_s,  lse = M + log2 sum_s 2^(lse_s - M),
//   o = sum_s 2^(lse_s - lse) * o_s,
//
// the combine segment of gqa_decode_splitkv in "decode_attention_splitkv.py"
// (TileLang tutorial, ch. 18), with the weight of split s for a head applied
// to that head's row, and the merge of "04_flash_decoding.py" (CS349E
// lecture 11), demo 1. One wave per (sequence, head): lanes first reduce the
// LSEs (max, then sum of 2^(lse_s - M)), then stream the fp32 partial rows
// with coalesced loads, D/64 dims per lane when D >= 64, otherwise several
// splits side by side; the output is rounded to the input dtype.
#include "fd_split.h"

namespace fd {

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int mask = 1; mask < kWave; mask <<= 1) x = fmaxf(x, __shfl_xor(x, mask));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int mask = 1; mask < kWave; mask <<= 1) x += __shfl_xor(x, mask);
  return x;
}

template <int DT, int D>
__global__ __launch_bounds__(kWave) void combine_kernel(CombineArgs a) {
  constexpr int DPL = D >= kWave ? D / kWave : 1;  // dims per lane
  constexpr int LPS = D / DPL;                     // lanes per partial row
  constexpr int SPW = kWave / LPS;                 // splits read side by side
  const int lane = threadIdx.x;
  const int bh = blockIdx.x;
  const int b = bh / a.heads;
  const int h = bh % a.heads;
  const int ns = a.num_splits;
  const float* lse = a.lse + (int64_t)b * ns * a.heads + h;  // stride heads
  const float* op = a.opart + (int64_t)bh * ns * D;

  float mx = kNegInf;
  for (int s = lane; s < ns; s += kWave) mx = fmaxf(mx, lse[(int64_t)s * a.heads]);
  mx = wave_max(mx);

  const int sg = lane / LPS;
  const int dl = lane % LPS;
  float acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.0f;

  if (mx != kNegInf) {
    float tot = 0.0f;
    for (int s = lane; s < ns; s += kWave) tot += fast_exp2(lse[(int64_t)s * a.heads] - mx);
    tot = wave_sum(tot);
    const float lse_all = mx + fast_log2(tot);
    int s = sg;
    // four splits in flight per lane group
    for (; s + 3 * SPW < ns; s += 4 * SPW) {
      float w[4];
      float v[4][DPL];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        w[u] = fast_exp2(lse[(int64_t)(s + u * SPW) * a.heads] - lse_all);
#pragma unroll
        for (int e = 0; e < DPL; ++e) v[u][e] = op[(int64_t)(s + u * SPW) * D + dl * DPL + e];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[e] = __builtin_fmaf(w[u], v[u][e], acc[e]);
    }
    for (; s < ns; s += SPW) {
      const float w = fast_exp2(lse[(int64_t)s * a.heads] - lse_all);
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] = __builtin_fmaf(w, op[(int64_t)s * D + dl * DPL + e], acc[e]);
    }
  }
#pragma unroll
  for (int mask = LPS; mask < kWave; mask <<= 1)
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] += __shfl_xor(acc[e], mask);
  if (sg == 0) {
#pragma unroll
    for (int e = 0; e < DPL; ++e) store_out<DT>(a.out, (int64_t)bh * D + dl * DPL + e, acc[e]);
  }
}

template <int DT>
static hipError_t launch_combine_dt(const CombineArgs& a, int dim, hipStream_t s) {
  dim3 grid((unsigned)(a.batch * a.heads));
  dim3 block(kWave);
  switch (dim) {
    case 16: hipLaunchKernelGGL((combine_kernel<DT, 16>), grid, block, 0, s, a); break;
    case 32: hipLaunchKernelGGL((combine_kernel<DT, 32>), grid, block, 0, s, a); break;
    case 64: hipLaunchKernelGGL((combine_kernel<DT, 64>), grid, block, 0, s, a); break;
    case 128: hipLaunchKernelGGL((combine_kernel<DT, 128>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, int dtype, int dim, hipStream_t s) {
  switch (dtype) {
    case DT_F32: return launch_combine_dt<DT_F32>(a, dim, s);
    case DT_F16: return launch_combine_dt<DT_F16>(a, dim, s);
    case DT_BF16: return launch_combine_dt<DT_BF16>(a, dim, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fd
