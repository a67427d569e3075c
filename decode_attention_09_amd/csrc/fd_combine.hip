// Combine kernel of flash decoding for gfx950, the second launch: merges
// the per-split normalised partial outputs with their base-2 log-sum-exps
// into the output.
#include "fd_split.h"

namespace fd {

// The LSE merge of one (sequence, head) by a workgroup of NWAVES waves:
//   M = max_s lse_s, lse = M + log2 sum_s 2^(lse_s - M),
//   o = sum_s 2^(lse_s - lse) * o_s,   rounded to the dtype,
// the combine segment of gqa_decode_splitkv in "decode_attention_splitkv.py"
// (TileLang tutorial, ch. 18), with the weight of split s for a head applied
// to that head's row, and the merge of "04_flash_decoding.py" (CS349E
// lecture 11), demo 1. Every thread first helps reduce the LSEs through
// LDS; then each wave streams a strided subset of the partial rows (SPW rows
// side by side, D/64 dims per lane when D >= 64) and the waves' sums meet in
// LDS. All threads of the workgroup must call it (it synchronises).
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

template <int DT, int D, int NWAVES>
__device__ __forceinline__ void combine_head(const float* opart, const float* lse_base, void* out,
                                             int heads, int ns, int b, int h) {
  constexpr int NT = kWave * NWAVES;
  constexpr int DPL = D >= kWave ? D / kWave : 1;  // dims per lane
  constexpr int LPS = D / DPL;                     // lanes per partial row
  constexpr int SPW = kWave / LPS;                 // rows a wave reads side by side
  constexpr int RPG = SPW * NWAVES;                // rows the group reads side by side
  __shared__ float red[NWAVES];
  __shared__ float part[NWAVES][D];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int64_t bh = (int64_t)b * heads + h;
  const float* lse = lse_base + (int64_t)b * ns * heads + h;  // split stride = heads
  const float* op = opart + bh * ns * D;

  float mx = kNegInf;
  for (int s = tid; s < ns; s += NT) mx = fmaxf(mx, lse[(int64_t)s * heads]);
  mx = wave_max(mx);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  mx = red[0];
#pragma unroll
  for (int w = 1; w < NWAVES; ++w) mx = fmaxf(mx, red[w]);
  __syncthreads();

  const int sg = lane / LPS;
  const int dl = lane % LPS;
  float acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.0f;

  if (mx != kNegInf) {  // uniform: every split empty -> zero row
    float tot = 0.0f;
    for (int s = tid; s < ns; s += NT) tot += fast_exp2(lse[(int64_t)s * heads] - mx);
    tot = wave_sum(tot);
    if (lane == 0) red[wave] = tot;
    __syncthreads();
    tot = 0.0f;
#pragma unroll
    for (int w = 0; w < NWAVES; ++w) tot += red[w];
    const float lse_all = mx + fast_log2(tot);
    int s = wave * SPW + sg;
    for (; s + 3 * RPG < ns; s += 4 * RPG) {
      float wt[4];
      float v[4][DPL];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        wt[u] = fast_exp2(lse[(int64_t)(s + u * RPG) * heads] - lse_all);
#pragma unroll
        for (int e = 0; e < DPL; ++e)
          v[u][e] = op[(int64_t)(s + u * RPG) * D + dl * DPL + e];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[e] = __builtin_fmaf(wt[u], v[u][e], acc[e]);
    }
    for (; s < ns; s += RPG) {
      const float wt = fast_exp2(lse[(int64_t)s * heads] - lse_all);
#pragma unroll
      for (int e = 0; e < DPL; ++e)
        acc[e] = __builtin_fmaf(wt, op[(int64_t)s * D + dl * DPL + e], acc[e]);
    }
  }
#pragma unroll
  for (int mask = LPS; mask < kWave; mask <<= 1)
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] += __shfl_xor(acc[e], mask);
  if (sg == 0) {
#pragma unroll
    for (int e = 0; e < DPL; ++e) part[wave][dl * DPL + e] = acc[e];
  }
  __syncthreads();
  for (int d = tid; d < D; d += NT) {
    float o = part[0][d];
#pragma unroll
    for (int w = 1; w < NWAVES; ++w) o += part[w][d];
    store_out<DT>(out, bh * D + d, o);
  }
}

constexpr int kCombineWaves = 4;

// One workgroup of four waves per (sequence, head).
template <int DT, int D>
__global__ __launch_bounds__(kWave* kCombineWaves) void combine_kernel(CombineArgs a) {
  const int bh = blockIdx.x;
  combine_head<DT, D, kCombineWaves>(a.opart, a.lse, a.out, a.heads, a.num_splits,
                                     bh / a.heads, bh % a.heads);
}

template <int DT>
static hipError_t launch_combine_dt(const CombineArgs& a, int dim, hipStream_t s) {
  dim3 grid((unsigned)(a.batch * a.heads));
  dim3 block(kWave * kCombineWaves);
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
