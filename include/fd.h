/*
 * fd.h -- C ABI of libfd: single-query split-KV decode attention
 * ("flash decoding") for AMD Instinct MI355X (gfx950).
 *
 * What is computed. For every sequence b and query head h of one decode
 * step, with G = heads / kv_heads and KV head j = h / G:
 *
 *     o[b,h,:] = softmax_t( scale * q[b,h,:] . K[b,t,j,:] ) V[b,t,j,:],
 *                t in [0, L_b),  L_b = cu_seqlens_k[b+1] - cu_seqlens_k[b].
 *
 * The KV axis of each (b, j) is cut into num_splits proportional segments
 * [L_b*s/num_splits, L_b*(s+1)/num_splits) (integer division). A first
 * kernel computes, per segment, the normalised partial output and its
 * log-sum-exp, with the G query heads of a group packed so one read of a
 * K/V row serves all of them; a second kernel merges the segments exactly
 * with log-sum-exp weights.
 *
 * Sources:
 *   - "decode_attention_splitkv.py" (TileLang tutorial, ch. 18):
 *     gqa_decode_splitkv -- GQA packing, cu_seqlens_k varlen addressing,
 *     proportional split bounds, split epilogue (o_s, base-2 LSE), combine
 *     segment; its docstring's rule that every split must hold >= 1 key.
 *   - "flash_decode_splitk.py" (MiniInfer): flash_decode_splitk host checks
 *     (supported head dims, positive KV length, default scale 1/sqrt(dim),
 *     default split count), output cast back to the input dtype.
 *   - "04_flash_decoding.py" (CS349E lecture 11), demos 1 and 4: the exact
 *     LSE merge, and choosing the split count so the number of workgroups is
 *     one to a few times the number of compute units (wave quantisation).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are device pointers, owned by the caller, and must
 *     be 16-byte aligned. The library allocates no device memory and keeps
 *     no per-call state; calls are asynchronous on `stream` (a hipStream_t
 *     passed as void*, NULL = the default stream), never synchronise and
 *     record no memset, so they can be captured in a HIP graph. The first
 *     call of a configuration on a device queries device and kernel
 *     attributes (cached afterwards): make it outside the capture.
 *   - Element type `dtype` (FD_F32, FD_F16, FD_BF16) applies to q, k, v and
 *     out. Scores, the softmax statistics and all accumulation are fp32;
 *     for fp16/bf16 the probabilities are rounded to dtype (round to
 *     nearest even) for the P.V products, which accumulate in fp32; out is
 *     rounded to dtype (round-to-nearest-even).
 *   - Return value: FD_OK or an FD_ERR_* code. Argument checks run on the
 *     host before anything is launched; a failed check launches nothing and
 *     leaves every buffer untouched.
 *   - cu_seqlens_k lives on the device and is never read by the host, so
 *     the device path cannot check `num_splits <= L_b`. A split that holds
 *     no key contributes nothing (its LSE is -inf, its partial output 0),
 *     and a sequence with L_b = 0 yields an all-zero output row. Callers
 *     should pick num_splits with fd_plan_splits, which enforces the rule.
 */
#ifndef FD_H_
#define FD_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of q, k, v, out. */
enum { FD_F32 = 0, FD_F16 = 1, FD_BF16 = 2 };

/* Status codes. */
enum {
  FD_OK = 0,
  FD_ERR_INVALID_ARG = 1,  /* null pointer, bad size, stride or alignment */
  FD_ERR_UNSUPPORTED = 2,  /* dim not in {16,32,64,128}, dtype, group > 64 */
  FD_ERR_EMPTY_SPLIT = 3,  /* planner: some sequence has no key */
  FD_ERR_HIP = 4,          /* a HIP runtime call or launch failed */
  FD_ERR_SCRATCH = 5       /* fd_decode_attention_noalloc: the call's partials
                              need more than FD_NOALLOC_SCRATCH_BYTES */
};

/* Limits. */
#define FD_MAX_SPLITS 16384
#define FD_MAX_GROUP 64

/*
 * Where the K/V row of sequence b, key t, KV head j starts, in elements:
 *
 *     b*batch_stride + cu_seqlens_k[b]*cu_stride + t*token_stride + j*head_stride
 *
 * Packed varlen [total_kv, kv_heads, dim] (decode_attention_splitkv.py,
 * shape_kv):        {0, dim, kv_heads*dim, kv_heads*dim}
 * Padded [batch, kv_heads, max_len, dim] (flash_decode_splitk.py's
 * [batch, heads, seqlen, dim]): {kv_heads*max_len*dim, max_len*dim, dim, 0}
 * Padded [batch, max_len, kv_heads, dim]:
 *                   {max_len*kv_heads*dim, dim, kv_heads*dim, 0}
 * (a view into a larger cache uses that cache's strides).
 *
 * Field order: batch_stride, head_stride, token_stride, cu_stride. All are
 * >= 0, token_stride >= dim, every stride*element_size is a multiple of 16
 * bytes, and token_stride*element_size <= 8 MiB (offsets inside one tile of
 * keys are 32-bit); otherwise FD_ERR_INVALID_ARG. K and V share the layout.
 * NULL means packed.
 */
typedef struct fd_kv_layout {
  int64_t batch_stride;
  int64_t head_stride;
  int64_t token_stride;
  int64_t cu_stride;
} fd_kv_layout;

/*
 * fd_plan_splits -- choose num_splits for a batch (host only, no device
 * access unless num_cus == 0).
 *
 *   seqlens_host  int32[batch] KV lengths on the host.
 *   num_cus       compute units to plan for; 0 = query the current device.
 *   max_splits    upper bound on the result (<= 0 means FD_MAX_SPLITS).
 *   *num_splits_out  receives the choice.
 *
 * Rule (04_flash_decoding.py, demo 4; flash_decode_splitk.py's floor of
 * 256 keys per split; decode_attention_splitkv.py's non-empty rule): among
 * split counts that leave every split >= 1 key and the longest sequence
 * >= 256 keys per split, take the one with the least modelled call time
 * (fd_plan_time_us). Ties go to fewer splits. When the calling thread's
 * schedule is FD_SCHED_STEAL (fd_set_schedule) and the call would run the
 * matrix-core kernel (head dim 128), the result is instead the steal
 * layout's partial-slot count, nsh * 4 with nsh = max(1, num_cus / units)
 * shares per unit (units = batch * kv_heads * ceil(group / 8)), provided
 * the longest sequence gives every share at least 1024 keys.
 * Returns FD_ERR_EMPTY_SPLIT if some length is < 1, FD_ERR_INVALID_ARG for
 * bad sizes, FD_ERR_HIP if the device query fails.
 */
int fd_plan_splits(int batch, int heads, int kv_heads, int dim, int dtype,
                   const int32_t* seqlens_host, int num_cus, int max_splits,
                   int* num_splits_out);

/*
 * fd_plan_schedule -- the schedule (fd_set_schedule) and split count the
 * library recommends for a batch (host only, arguments as fd_plan_splits).
 * Ragged batches (longest sequence >= 1.5x the shortest): FD_SCHED_QUEUE
 * with about 4 segments per compute unit, num_splits = round(4 * num_cus /
 * units) (units = batch * kv_heads * ceil(group / 8)), capped by the
 * shortest sequence, 256 keys per split of the longest and max_splits,
 * where that fills the device. Otherwise FD_SCHED_STEAL with the steal
 * layout's slot count (see fd_plan_splits) when the call would run the
 * matrix-core kernel at head dim 128, the longest sequence is at most 4x
 * the shortest and each share of the longest sequence streams >= 12 MB of
 * K and V; else FD_SCHED_STATIC with fd_plan_splits's count. The rules are
 * MI355X's measured ones (the queue at 4 segments per CU was the fastest
 * option or within 1.3 % of it on every ragged batch tried; near-uniform
 * Llama-3.1-8B-shaped calls of 4-17 GB with such shares run 1-8 % faster
 * under the steal schedule, shorter shares slower). The caller sets the
 * schedule with fd_set_schedule before the call. Errors as fd_plan_splits.
 */
int fd_plan_schedule(int batch, int heads, int kv_heads, int dim, int dtype,
                     const int32_t* seqlens_host, int num_cus, int max_splits,
                     int* schedule_out, int* num_splits_out);

/*
 * fd_plan_time_us -- the planner's modelled time, in microseconds, of one
 * fd_decode_attention call (split launch plus, for num_splits > 1, the
 * combine launch) with this split count: the time column of the split-count
 * table of 04_flash_decoding.py (demo 4), for MI355X. The workgroups
 * (batch * kv_heads * ceil(group / 8) * num_splits) run in rounds of
 * min(num_cus, remaining); a round costs a fixed workgroup time plus its
 * largest segment's K/V bytes at a per-byte time that grows with the number
 * of workgroups streaming at once; unequal lengths take the average load
 * plus the largest segment (list-scheduling bound). The constants were
 * fitted to measured MI355X calls (relative RMS error 4.7 %). Same
 * arguments as fd_plan_splits; returns a negative value on bad arguments.
 */
double fd_plan_time_us(int batch, int heads, int kv_heads, int dim, int dtype,
                       const int32_t* seqlens_host, int num_cus, int num_splits);

/*
 * fd_workspace_bytes -- size of the workspace for a call with these
 * sizes (0 on overflow or bad sizes). Layout:
 *   Opart [batch, heads, num_splits, dim]  fp32, normalised partial outputs o_s
 *   LSE   [batch, num_splits, heads]       fp32, log2(sum_t 2^(s2_t)) of split
 *                                           s, s2_t = scale*log2(e)*q.k_t
 *   control                                256 bytes holding the claim counter
 *                                           of a queue-scheduled launch
 *                                           (fd_set_schedule), then int32
 *                                           [batch*heads] arrival counters of
 *                                           fused calls (fd_set_combine),
 *                                           padded to a multiple of 256 bytes,
 *                                           then 4096 uint64 share words of a
 *                                           steal-scheduled call
 * LSE starts at the first 256-byte boundary after Opart, the control block
 * at the first 256-byte boundary after LSE. The shapes follow part_shape /
 * lse_shape of decode_attention_splitkv.py, in fp32. Its contents before a
 * call do not matter, except for the arrival counters of a fused call,
 * which must be zero (queue- and steal-scheduled calls zero their own
 * counter and words with a kernel launched just before the split launch).
 */
size_t fd_workspace_bytes(int batch, int heads, int num_splits, int dim);

/*
 * fd_decode_attention -- the whole hot path: split kernel + LSE combine.
 *
 *   q             [batch, heads, dim] dtype, contiguous.
 *   k, v          KV cache, addressed by `layout` (NULL = packed).
 *   cu_seqlens_k  int32[batch+1] device array of non-decreasing offsets.
 *   num_splits    1..FD_MAX_SPLITS. With 1, the split kernel writes `out`
 *                 directly and `workspace` may be NULL.
 *   scale         softmax scale on q.k in natural-exp units (any finite
 *                 value; 1/sqrt(dim) is the usual choice).
 *   out           [batch, heads, dim] dtype, fully overwritten.
 *   workspace     fd_workspace_bytes(...) bytes of device memory, or NULL
 *                 when num_splits == 1. Contents on return: the partials.
 *                 Calls that run concurrently must not share a workspace.
 *   stream        hipStream_t as void*.
 */
int fd_decode_attention(const void* q, const void* k, const void* v,
                        const int32_t* cu_seqlens_k, int batch, int heads,
                        int kv_heads, int dim, int num_splits, float scale,
                        void* out, void* workspace, void* stream, int dtype,
                        const fd_kv_layout* layout);

/*
 * fd_decode_split -- first launch only: writes Opart and LSE for every
 * (b, h, split) into `workspace` (required, for any num_splits >= 1).
 * Same arguments as fd_decode_attention minus `out`.
 */
int fd_decode_split(const void* q, const void* k, const void* v,
                    const int32_t* cu_seqlens_k, int batch, int heads,
                    int kv_heads, int dim, int num_splits, float scale,
                    void* workspace, void* stream, int dtype,
                    const fd_kv_layout* layout);

/*
 * fd_decode_combine -- second launch only: merges the Opart/LSE workspace
 * written by fd_decode_split (or any producer of the same layout, e.g. the
 * shards of a sequence-parallel split) into out [batch, heads, dim] dtype:
 * M = max_s LSE_s, lse = M + log2 sum_s 2^(LSE_s - M),
 * out = sum_s 2^(LSE_s - lse) * Opart_s (combine segment of
 * decode_attention_splitkv.py). Rows whose splits are all empty get 0.
 */
int fd_decode_combine(const void* workspace, int batch, int heads, int dim,
                      int num_splits, void* out, void* stream, int dtype);

/*
 * The second workspace format, that of _splitk_stage1_kernel and
 * _splitk_reduce_kernel in "flash_decode_splitk.py" (MiniInfer):
 *
 *   - split bounds are ceil-equal: with size = ceil(L_b / num_splits),
 *     split s covers keys [s*size, min(s*size + size, L_b)); splits that
 *     start at or past L_b are empty, which is allowed (any num_splits in
 *     1..FD_MAX_SPLITS, whatever the lengths);
 *   - every split leaves its unnormalised state, with s2_t = scale *
 *     log2(e) * q.k_t the base-2 scaled scores of its keys:
 *       m_s   = max_t s2_t                      (-inf for an empty split)
 *       l_s   = sum_t 2^(s2_t - m_s)            (0 for an empty split)
 *       acc_s = sum_t 2^(s2_t - m_s) * v_t      (0 for an empty split)
 *   - the combine rescales to M = max_s m_s:
 *       o = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s,
 *     and writes zeros for a row whose splits are all empty.
 *
 * The result is the same attention as fd_decode_attention's (same
 * tolerances); only the bounds and the partials differ. Arguments,
 * alignment, layout, ownership and error codes are those of the
 * corresponding functions above.
 *
 * fd_workspace_bytes_unnorm -- fp32 workspace of the unnormalised format:
 *   ACC [batch, heads, num_splits, dim]   acc_s
 *   M   [batch, heads, num_splits]        m_s   (first 256-B boundary after ACC)
 *   L   [batch, heads, num_splits]        l_s   (first 256-B boundary after M)
 * the layouts of ACC_BUF ([bh, ns, dim]) and M_BUF / L_BUF ([bh, ns]). 0 on
 * bad sizes.
 */
size_t fd_workspace_bytes_unnorm(int batch, int heads, int num_splits, int dim);

/* fd_decode_split_unnorm -- split launch only, writing (ACC, M, L) into
 * `workspace` (fd_workspace_bytes_unnorm bytes, required). */
int fd_decode_split_unnorm(const void* q, const void* k, const void* v,
                           const int32_t* cu_seqlens_k, int batch, int heads,
                           int kv_heads, int dim, int num_splits, float scale,
                           void* workspace, void* stream, int dtype,
                           const fd_kv_layout* layout);

/* fd_decode_combine_unnorm -- combine launch only, from an (ACC, M, L)
 * workspace into out [batch, heads, dim] dtype. */
int fd_decode_combine_unnorm(const void* workspace, int batch, int heads, int dim,
                             int num_splits, void* out, void* stream, int dtype);

/* fd_decode_attention_unnorm -- split + combine in this format. With
 * num_splits == 1 one launch writes `out` directly and `workspace` may be
 * NULL (one split is the whole sequence under either bound rule). */
int fd_decode_attention_unnorm(const void* q, const void* k, const void* v,
                               const int32_t* cu_seqlens_k, int batch, int heads,
                               int kv_heads, int dim, int num_splits, float scale,
                               void* out, void* workspace, void* stream, int dtype,
                               const fd_kv_layout* layout);

/*
 * fd_set_kernel_path -- which split kernel later calls made from the calling
 * thread launch (a per-thread setting, for benchmarks and tests that compare
 * the kernels; other threads and calls already enqueued are unaffected; a
 * new thread starts at FD_PATH_AUTO). FD_PATH_VALU: vector-ALU dot products (v_dot2 / FMA) for
 * QK^T and PV everywhere. FD_PATH_MFMA: QK^T on the matrix cores
 * (v_mfma_f32_16x16x32_{f16,bf16}, v_mfma_f32_16x16x4_f32) wherever that
 * kernel exists -- head dim 128 -- and the VALU kernel elsewhere. FD_PATH_AUTO (the
 * default): the library's measured choice. FD_PATH_UNPACKED: the VALU
 * kernel with one query head per workgroup, so each K/V row is read once
 * per query head instead of once per GQA group -- the unpacked,
 * FlashAttention-2-style decode that 04_flash_decoding.py (demos 2-3)
 * compares flash decoding against; a comparator, never a default. All paths
 * compute the same function to the same tolerances. Returns the previous
 * setting, or -1 (setting unchanged) for an unknown value.
 */
enum { FD_PATH_AUTO = 0, FD_PATH_VALU = 1, FD_PATH_MFMA = 2, FD_PATH_UNPACKED = 3 };
int fd_set_kernel_path(int path);

/*
 * fd_set_schedule -- how later split launches from the calling thread hand
 * segments to workgroups (a per-thread setting, like fd_set_kernel_path).
 * FD_SCHED_STATIC: one workgroup per segment, in the fixed order of the
 * grid. FD_SCHED_QUEUE: as many workgroups as the device holds at once;
 * each takes one segment, then claims the next unprocessed one from a
 * counter in the workspace's control block (zeroed by a one-thread kernel
 * launched just before, on the same stream), so compute units that stream
 * faster process more segments. FD_SCHED_AUTO (the default): the library's
 * measured choice. The segments, their bounds and every partial are the
 * same under the static and queue schedules, so their results are bitwise
 * identical; the queue applies to launches with a normalised-format
 * workspace (fd_decode_attention with a workspace,
 * fd_decode_attention_noalloc, fd_decode_split) and is ignored elsewhere.
 * FD_SCHED_STEAL (normalised-format launches on the matrix-core kernel
 * with num_splits > 1; others run the static schedule): the keys of each
 * (sequence, KV
 * head) unit are cut into nsh proportional shares, one workgroup each,
 * where nsh is the largest divisor of num_splits <= num_splits / 2 with
 * units * nsh <= the device's compute units and cap = num_splits / nsh - 1
 * in 1..15 (none: static schedule). Share r owns partial slots
 * r*(1+cap) .. r*(1+cap)+cap. Its workgroup streams the share in chunks it
 * claims one ahead from the share's word; a workgroup that is done takes
 * the back half of the unclaimed chunks of the share that has the most,
 * up to cap times per share, each take one partial in the next slot; slots
 * no run used hold LSE -inf and zeros. The same attention, but the key
 * ranges merged depend on timing, so results vary by rounding between
 * calls. The partials fd_decode_split leaves are then these slots, not
 * the proportional splits; fd_decode_combine merges them alike (a
 * fused-combine call runs the static schedule). fd_plan_splits gives the
 * slot count. Returns the previous
 * setting, or -1 (unchanged) for an unknown value.
 */
enum { FD_SCHED_AUTO = 0, FD_SCHED_STATIC = 1, FD_SCHED_QUEUE = 2, FD_SCHED_STEAL = 3 };
int fd_set_schedule(int sched);

/*
 * fd_set_combine -- where later fd_decode_attention calls made from the
 * calling thread merge the partials (a per-thread setting, like
 * fd_set_kernel_path). FD_COMBINE_SEPARATE (the default): the second
 * launch, fd_decode_combine's kernel. FD_COMBINE_FUSED: one launch -- the
 * per-kernel fixed cost that "04_flash_decoding.py" (CS349E lecture 11,
 * demo 3) counts twice for flash decoding is paid once: each split
 * workgroup stores its partials and counts itself in at the arrival
 * counter of its (sequence, KV head) in the workspace's control block (an
 * agent-scope acq_rel fetch_add); the last of the num_splits workgroups
 * merges them into `out` with the same LSE formula and sets the counter
 * back to zero. Requirements of the fused mode: the arrival counters of
 * the workspace must be zero before the call -- zero the whole workspace
 * once when it is allocated; every fused call leaves them zero, and
 * unfused calls never touch them. It applies to fd_decode_attention with
 * num_splits > 1 (one split is a single launch anyway); the unnormalised
 * format and fd_decode_attention_noalloc always use the second launch.
 * Results equal the two-launch path's within the stated tolerances (the
 * merge sums the splits in a different order). Returns the previous
 * setting, or -1 (unchanged) for an unknown value.
 */
enum { FD_COMBINE_SEPARATE = 0, FD_COMBINE_FUSED = 1 };
int fd_set_combine(int mode);

/*
 * fd_decode_attention_noalloc -- fd_decode_attention for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. Same kernels, arguments and result as
 * fd_decode_attention, except that there is no workspace argument: the
 * partials (fd_workspace_bytes(batch, heads, num_splits, dim) bytes) go to a
 * static device array of FD_NOALLOC_SCRATCH_BYTES bytes that the library
 * holds on every GPU it runs on until the process ends. The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine); the caller
 * still owns q, k, v, cu_seqlens_k and out.
 *
 *   - A call whose partials need more than FD_NOALLOC_SCRATCH_BYTES returns
 *     FD_ERR_SCRATCH before launching anything (fd_last_error() says how
 *     much it needed); num_splits == 1 needs none.
 *   - Every call on one GPU uses that GPU's one array, whatever the stream:
 *     calls that overlap in time on one GPU (concurrent streams, graph
 *     replays running side by side) race on it and must be serialised by
 *     the caller. The array keeps the last call's partials; nothing in it
 *     needs to start at zero (each call writes every partial it reads).
 *   - The first call on a device looks up that device's copy of the array
 *     (hipGetSymbolAddress) and caches it: make that call outside a graph
 *     capture.
 */
#define FD_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int fd_decode_attention_noalloc(const void* q, const void* k, const void* v,
                                const int32_t* cu_seqlens_k, int batch, int heads,
                                int kv_heads, int dim, int num_splits, float scale,
                                void* out, void* stream, int dtype,
                                const fd_kv_layout* layout);

/* Human-readable name of a status code (static string, never NULL). */
const char* fd_status_string(int status);

/* Last error text recorded by this thread when FD_ERR_HIP or FD_ERR_SCRATCH
 * was returned (static per-thread buffer, "" if none). */
const char* fd_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FD_H_ */
