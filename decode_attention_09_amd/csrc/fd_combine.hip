// Combine kernel of flash decoding for gfx950, the second launch: merges
// the per-split normalised partial outputs with their base-2 log-sum-exps
// into the output.
#include "fd_split.h"

namespace fd {

// The merge of one (sequence, head), or of D of its dims, by a workgroup of
// NWAVES waves.
//
// Normalised format (UNNORM = false), the combine segment of
// gqa_decode_splitkv in "decode_attention_splitkv.py" (TileLang tutorial,
// ch. 18) and the merge of "04_flash_decoding.py" (CS349E lecture 11),
// demo 1, with the weight of split s for a head applied to that head's row:
//   M = max_s lse_s, lse = M + log2 sum_s 2^(lse_s - M),
//   o = sum_s 2^(lse_s - lse) * o_s.
// Unnormalised format (UNNORM = true), _splitk_reduce_kernel of
// "flash_decode_splitk.py" (MiniInfer):
//   M = max_s m_s, alpha_s = 2^(m_s - M),
//   o = sum_s alpha_s acc_s / sum_s alpha_s l_s.
// Either way o is rounded to the dtype; a row whose splits are all empty
// (every key -inf) is written as zeros.
//
// key[s * kst] is lse_s or m_s, lw[s * kst] is l_s (unnormalised format),
// op[s * RS + d] the partial row of split s (RS: the head dim). Each wave owns a strided subset
// of the partial rows (SPW rows side by side, D/64 dims per lane when
// D >= 64). Every load the merge needs is issued up front -- one key (and l)
// per thread for the max and the sum, and the first KR partial rows of each
// lane group with their keys -- so the merge waits for memory once; rows
// beyond KR (many splits) are read after the reductions. The waves' maxima,
// sums and row sums meet in LDS. All threads of the workgroup must call it
// (it synchronises).
template <int DT, int D, int NWAVES, bool UNNORM, int RS = D, int KR = 8>
__device__ __forceinline__ void combine_head(const float* op, const float* key, const float* lw,
                                             int64_t kst, int ns, void* out, int64_t obase) {
  // D: dims this workgroup merges; RS: row stride of the partials (the head
  // dim); KR: rows per lane group held in registers; out + obase: the
  // first output element of those D dims.
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
  const int sg = lane / LPS;
  const int dl = lane % LPS;
  const int s0 = wave * SPW + sg;  // first partial row of this lane group

  // every load up front
  const float k_own = tid < ns ? key[(int64_t)tid * kst] : kNegInf;
  const float l_own = UNNORM && tid < ns ? lw[(int64_t)tid * kst] : 0.0f;
  float pk[KR], pv[KR][DPL];
#pragma unroll
  for (int k = 0; k < KR; ++k) {
    const int s = s0 + k * RPG;
    const bool in = s < ns;
    pk[k] = in ? key[(int64_t)s * kst] : kNegInf;
#pragma unroll
    for (int e = 0; e < DPL; ++e) pv[k][e] = in ? op[(int64_t)s * RS + dl * DPL + e] : 0.0f;
  }

  float mx = k_own;
  for (int s = tid + NT; s < ns; s += NT) mx = fmaxf(mx, key[(int64_t)s * kst]);
  mx = across_groups<1>(mx, OpMax{});
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  mx = red[0];
#pragma unroll
  for (int w = 1; w < NWAVES; ++w) mx = fmaxf(mx, red[w]);
  __syncthreads();

  float acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.0f;

  if (mx != kNegInf) {  // uniform: every split empty -> zero row
    // tot = sum_s 2^(key_s - mx) (times l_s in the unnormalised format)
    float tot = k_own == kNegInf ? 0.0f : fast_exp2(k_own - mx) * (UNNORM ? l_own : 1.0f);
    for (int s = tid + NT; s < ns; s += NT) {
      const float x = fast_exp2(key[(int64_t)s * kst] - mx);
      tot += UNNORM ? x * lw[(int64_t)s * kst] : x;
    }
    tot = across_groups<1>(tot, OpAdd{});
    if (lane == 0) red[wave] = tot;
    __syncthreads();
    tot = 0.0f;
#pragma unroll
    for (int w = 0; w < NWAVES; ++w) tot += red[w];
    // weight of split s: 2^(key_s - lse) = 2^(key_s - mx) / tot, written
    // as the page's formula of each format
    const float lse_all = mx + fast_log2(tot);
    const float inv_tot = 1.0f / tot;
    auto weight = [&](float ks) {
      return UNNORM ? fast_exp2(ks - mx) * inv_tot : fast_exp2(ks - lse_all);
    };
#pragma unroll
    for (int k = 0; k < KR; ++k) {
      const float wt = weight(pk[k]);  // 0 for rows past ns
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] = __builtin_fmaf(wt, pv[k][e], acc[e]);
    }
    int s = s0 + KR * RPG;
    for (; s + 3 * RPG < ns; s += 4 * RPG) {
      float wt[4];
      float v[4][DPL];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        wt[u] = weight(key[(int64_t)(s + u * RPG) * kst]);
#pragma unroll
        for (int e = 0; e < DPL; ++e)
          v[u][e] = op[(int64_t)(s + u * RPG) * RS + dl * DPL + e];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[e] = __builtin_fmaf(wt[u], v[u][e], acc[e]);
    }
    for (; s < ns; s += RPG) {
      const float wt = weight(key[(int64_t)s * kst]);
#pragma unroll
      for (int e = 0; e < DPL; ++e)
        acc[e] = __builtin_fmaf(wt, op[(int64_t)s * RS + dl * DPL + e], acc[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = across_groups<LPS>(acc[e], OpAdd{});
  if (sg == 0) {
#pragma unroll
    for (int e = 0; e < DPL; ++e) part[wave][dl * DPL + e] = acc[e];
  }
  __syncthreads();
  for (int d = tid; d < D; d += NT) {
    float o = part[0][d];
#pragma unroll
    for (int w = 1; w < NWAVES; ++w) o += part[w][d];
    store_out<DT>(out, obase + d, o);
  }
}

constexpr int kCombineWaves = 4;

// One workgroup of four waves per (sequence, head) and chunk of C of the
// head's D dims (C = 1: the whole head).
template <int DT, int D, int C, int KR>
__global__ __launch_bounds__(kWave* kCombineWaves) void combine_kernel(CombineArgs a) {
  constexpr int DC = D / C;
  const int64_t bh = blockIdx.x / C;
  const int c = (int)(blockIdx.x % C);
  const int ns = a.num_splits;
  const float* op = a.opart + bh * ns * D + c * DC;
  const int64_t obase = bh * D + c * DC;
  if (a.unnorm) {
    // m_s, l_s at [B, H, ns]
    combine_head<DT, DC, kCombineWaves, true, D, KR>(op, a.mbuf + bh * ns, a.lbuf + bh * ns, 1,
                                                     ns, a.out, obase);
  } else {
    // lse_s at [B, ns, H]: split stride = heads
    const int64_t b = bh / a.heads, h = bh % a.heads;
    combine_head<DT, DC, kCombineWaves, false, D, KR>(op, a.lse + b * ns * a.heads + h, nullptr,
                                                      a.heads, ns, a.out, obase);
  }
}

// Few (sequence, head) pairs with many splits leave most compute units idle
// and each workgroup reading its rows in several dependent rounds; then
// four workgroups share a head, 32 dims each, with every partial row loaded
// before the reductions. Measured on MI355X, per call: flash-decoding
// B1/64K (16 heads, 128 splits) 21.1 -> 19.2 us, B1/128K 31.8 -> 29.8 us,
// B2/32K (64 splits) 20.3 -> 19.6 us, Llama B1/64K at 128 splits
// 51.9 -> 49.8 us; at 32 splits or fewer, or more heads, no difference.
#ifndef FD_COMBINE_CHUNK_HEADS
#define FD_COMBINE_CHUNK_HEADS 64
#endif
#ifndef FD_COMBINE_CHUNK_MIN_SPLITS
#define FD_COMBINE_CHUNK_MIN_SPLITS 33
#endif

template <int DT, int D>
static void launch_combine_d(const CombineArgs& a, hipStream_t s) {
  const dim3 block(kWave * kCombineWaves);
  const int64_t bh = (int64_t)a.batch * a.heads;
  if constexpr (D == 128) {
    if (bh <= FD_COMBINE_CHUNK_HEADS && a.num_splits >= FD_COMBINE_CHUNK_MIN_SPLITS) {
      hipLaunchKernelGGL((combine_kernel<DT, D, 4, 16>), dim3((unsigned)(bh * 4)), block, 0, s, a);
      return;
    }
  }
  hipLaunchKernelGGL((combine_kernel<DT, D, 1, 8>), dim3((unsigned)bh), block, 0, s, a);
}

template <int DT>
static hipError_t launch_combine_dt(const CombineArgs& a, int dim, hipStream_t s) {
  switch (dim) {
    case 16: launch_combine_d<DT, 16>(a, s); break;
    case 32: launch_combine_d<DT, 32>(a, s); break;
    case 64: launch_combine_d<DT, 64>(a, s); break;
    case 128: launch_combine_d<DT, 128>(a, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// One thread zeroes the claim counter of the queue-scheduled split launch
// that follows on the same stream (stream order makes the zero visible to
// it). A kernel rather than a memset, so that a captured graph holds no
// memset node.
__global__ void queue_reset_kernel(int* queue) {
  if (threadIdx.x == 0) queue[0] = 0;
}

hipError_t launch_queue_reset(int* queue, hipStream_t s) {
  hipLaunchKernelGGL(queue_reset_kernel, dim3(1), dim3(kWave), 0, s, queue);
  return hipGetLastError();
}

__global__ void steal_reset_kernel(unsigned long long* words, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    words[i] = 0ull;
}

hipError_t launch_steal_reset(unsigned long long* words, int n, hipStream_t s) {
  const int block = 256;
  const int grid = n > 0 ? (n + block - 1) / block : 1;
  hipLaunchKernelGGL(steal_reset_kernel, dim3(grid < 64 ? grid : 64), dim3(block), 0, s, words,
                     n);
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
