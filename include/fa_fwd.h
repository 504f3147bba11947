/*
 * fa_fwd.h -- FlashAttention forward on MI355X (gfx950): the C ABI.
 *
 * Computes, per (batch or sequence, query head), the attention forward of the
 * aclnnFlashAttentionVarLenScoreV5 page (功能说明 -> 计算公式):
 *
 *     Attention = Softmax( Mask( scale * (Q K^T + Qrope Krope^T) + pse ), atten_mask ) * V
 *
 * with the optional per-head sink logit of the same section (m = max(sink,
 * max S); the denominator gains e^(sink - m)), and writes the per-row
 * softmax statistics softmaxMax = m and softmaxSum = l beside the output
 * (V5 parameter table, rows softmaxMaxOut / softmaxSumOut).
 *
 * The call is two-phase, as on both Ascend pages (aclnnFlashAttentionScore
 * page, 接口原型; V5 page, 函数原型): phase 1 validates the arguments on the
 * host and returns the workspace size and a plan; phase 2 enqueues the device
 * work on a HIP stream.
 *
 * Conventions
 *   - Every pointer inside an fa_tensor is a DEVICE address owned by the
 *     caller; the library never allocates, frees or reads device memory on the
 *     host.  Host arguments (descriptors, strings, out-pointers) are read only
 *     during the call.
 *   - Strides are in elements.  The last dimension of every tensor must have
 *     stride 1 except where noted.
 *   - Errors are returned as status codes; nothing is thrown across the ABI.
 *     fa_last_error_message() gives a human-readable reason for the last
 *     non-zero status returned on the calling thread.
 *   - All entry points are thread-safe; plans are immutable after phase 1.
 */
#ifndef FA_FWD_H
#define FA_FWD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of fa_tensor.dtype. */
typedef enum {
  FA_DTYPE_F32 = 0,
  FA_DTYPE_F16 = 1,
  FA_DTYPE_BF16 = 2,
  FA_DTYPE_U8 = 3,
  FA_DTYPE_BOOL = 4, /* one byte per element, 0 / 1 */
  FA_DTYPE_I32 = 5,
  FA_DTYPE_I64 = 6
} fa_dtype;

/* A strided view of device memory (the role of aclTensor on the Ascend pages:
 * shape, dtype, strides, device address).  ndim is 1..4; shape[i] >= 0;
 * stride[i] in elements; entries at index >= ndim are ignored. */
typedef struct {
  void* data;
  int32_t dtype; /* fa_dtype */
  int32_t ndim;
  int64_t shape[4];
  int64_t stride[4];
} fa_tensor;

/* Opaque execution plan (the role of aclOpExecutor). */
typedef struct fa_plan fa_plan;

typedef int32_t fa_status;

/* Status codes.  The first three carry the numbers of the pages' aclnn
 * return-code table (V5 page, 返回值: ACLNN_ERR_PARAM_NULLPTR 161001,
 * ACLNN_ERR_PARAM_INVALID 161002, ACLNN_ERR_INNER_NULLPTR 561103). */
#define FA_OK 0
#define FA_ERR_PARAM_NULLPTR 161001 /* a required pointer argument is NULL          */
#define FA_ERR_PARAM_INVALID 161002 /* dtype, layout string or tensor format invalid */
#define FA_ERR_UNSUPPORTED 561103   /* shape or attribute outside the supported range */
#define FA_ERR_WORKSPACE 561201     /* phase 2: workspace NULL or smaller than needed */
#define FA_ERR_RUNTIME 561202       /* phase 2: HIP launch / runtime error            */

/*
 * Phase 1: validate, plan, and report the device workspace size.
 *
 * Passages: V5 page, 函数原型 and the 参数说明 table (argument list and
 * meaning); aclnnFlashAttentionScore page, aclnnFlashAttentionScoreGetWorkspaceSize
 * 参数说明 (dense layouts BSH / SBH / BSND / BNSD); MindIE-SD
 * attention_forward_varlen page (int32 cu_seqlens with a leading 0, causal).
 *
 * Arguments (device tensors unless stated; NULL = absent for optional ones):
 *   query, key, value   q/k/v, one dtype of F32, F16, BF16.  Layout by
 *                       input_layout: BNSD [B,N,S,D], BSND [B,S,N,D],
 *                       BSH [B,S,N*D], SBH [S,B,N*D], TND [T,N,D].
 *                       Nq % Nkv == 0 (GQA / MQA: query head h reads kv
 *                       head h / (Nq/Nkv)); D(q) == D(k) >= D(v).
 *   query_rope, key_rope  optional, both or neither; F16 or BF16 equal to q's
 *                       dtype, same layout and sizes as query / key with their
 *                       own last dim Dr.  Adds Qrope Krope^T to the scores.
 *   real_shift          optional pse, q's dtype: the additive position bias
 *                       of the attention equation, added after the scale
 *                       (pseType 1; the V5 parameter table, row
 *                       realShiftOptional).  Dense: [B|1, N, Sq, Skv], last
 *                       dim contiguous, any other strides.  TND: 1-D, one
 *                       [N, Sq_i, Skv_i] block per sequence in sequence
 *                       order (reads beyond shape[0] return 0: the caller
 *                       keeps the length equal to sum_i N * Sq_i * Skv_i).
 *                       Not with query_rope / key_rope; the compressed
 *                       last-1024-rows form is not supported.  With a scale
 *                       of 0 the bias must stay below 2e8 in magnitude.
 *   atten_mask          optional U8/BOOL, nonzero = position EXCLUDED.
 *                       Dense: [B,N,Sq,Skv], [B,1,Sq,Skv], [1,1,Sq,Skv] or
 *                       [Sq,Skv] (any strides).  TND: a 2-D [S1,S2] matrix
 *                       read in sequence-local coordinates; positions outside
 *                       it count as excluded.  The mask is read only in KV
 *                       blocks that cross the preTokens/nextTokens window
 *                       boundary or the sequence end (sparse mode 0 requires
 *                       the mask to agree with the window); when the window
 *                       cuts nothing it is read everywhere.
 *   sink                optional F32 [Nq]: per-query-head sink logit, in
 *                       logit units (not scaled).  -inf equals no sink.
 *   cu_seqlens_q, cu_seqlens_kv  TND only (required there, NULL otherwise):
 *                       I32 [B+1], cumulative lengths with a leading 0,
 *                       non-decreasing, last entry == T of q / k.  Read by the
 *                       device in phase 2 only; zero-length sequences allowed.
 *   q_start_idx, kv_start_idx  optional HOST pointers to one int64 each (NULL
 *                       = 0): where this call's query rows and key rows start
 *                       in the whole sequence, for an outer split along the
 *                       sequence (V5 parameter table, rows qStartIdxOptional /
 *                       kvStartIdxOptional).  The causal and preTokens /
 *                       nextTokens tests then use global positions
 *                       i + q_start_idx and j + kv_start_idx; atten_mask stays
 *                       in the call's own coordinates.  Each in [0, 2^26].
 *   scale_value         finite, >= 0; multiplies both score terms.
 *   keep_prob           must be 1.0 (no dropout).
 *   pre_tokens, next_tokens  window: key j is kept for row i iff
 *                       -pre <= j - i <= next (inclusive), counted from the
 *                       start of each sequence.  Active only when atten_mask
 *                       is given or causal != 0; then pre + next' >= 0 is
 *                       required, next' = min(next, 0) under causal.
 *   head_num            Nq; must equal the query's N (splits H for BSH/SBH).
 *   input_layout        "BNSD" | "BSND" | "BSH" | "SBH" | "TND".
 *   inner_precise       0, 1 or 2; accepted, numerics are the same for all
 *                       (fp32 accumulation; rows with no kept key are defined).
 *   sparse_mode         must be 0.
 *   causal              nonzero: exclude j > i (top-left aligned).
 *   softmax_out_layout  NULL or "" or "same_as_input" (TND stats layout).
 *   softmax_max, softmax_sum  optional F32 outputs (NULL = not written):
 *                       dense [B,N,Sq,8]; TND [N,T,8] for "" and [T,N,8] for
 *                       "same_as_input".  All 8 trailing slots hold the same
 *                       per-row value: m = max(sink, max_j s_ij) in natural-log
 *                       units and l = sum_j e^(s_ij - m) (+ e^(sink - m)).
 *                       A row with no kept key gets m = -inf, l = 0 (or
 *                       m = sink, l = 1 with a finite sink).
 *   attention_out       output, q's dtype, q's layout with last dim Dv.  Rows
 *                       with no kept key are 0.  Rounded to nearest even.
 *   workspace_size      host out: bytes of device workspace phase 2 needs,
 *                       16-byte aligned parts: for TND with more than 256
 *                       sequences the tile prefix (4 (B+1) bytes) and a
 *                       32-byte tile-map entry per tile of the grid (up to
 *                       256 sequences the kernels find their tiles from
 *                       cu_seqlens_q themselves), then 8 (B+1) bytes of pse block
 *                       offsets with a TND real_shift; with atten_mask one
 *                       class byte per (mask slice, 128-row tile, 64-key
 *                       block), padded to 16; with a key split (below)
 *                       kv_splits x B x N x Sq x (Dv + 2) fp32 partial
 *                       results.  0 for a dense call without a mask or key
 *                       split.  The workspace must be 16-byte aligned.
 *   plan                host out: a new plan, to be released with
 *                       fa_plan_destroy().  It records the tensors' device
 *                       addresses; it may be executed any number of times.
 *
 * Kernel choice: a matrix-core kernel when q is F16/BF16, D is 64, 96 or 128,
 * Dr is 0 or 64, Dv == D (or, with no rope inputs and no real_shift,
 * D == Dv + 64, the last 64 dims of q and k then taking the rope part's
 * role) and every row start is 16-byte aligned (the
 * two-group one for dense Sq, Skv >= 1024 at D = 128 without rope or pse
 * whose window cuts at most the causal side or spans at least 2048 keys
 * (pre + next >= 2047), whose grid of 256-row tiles has at least 256
 * workgroups and whose K / V rows of one sequence span under 2 GiB, else the
 * four-wave one);
 * otherwise the generic one (fp32 dot products on the vector units).  The environment
 * variable FA_FWD_KERNEL = "mfma" | "pp" | "generic", read here, forces a
 * family for testing; forcing one the arguments do not fit returns
 * FA_ERR_UNSUPPORTED.  Key split: a dense four-wave grid of fewer than 512
 * workgroups (two per compute unit) runs up to 4 workgroups per query tile,
 * each over a contiguous range of at least 512 keys, and merges their fp32
 * partial results (the combination fa_fwd_merge states) in a second kernel;
 * FA_FWD_KV_SPLIT = 1..4 forces the number of ranges (1 = no split), other
 * values return FA_ERR_UNSUPPORTED.
 *
 * Returns FA_OK, FA_ERR_PARAM_NULLPTR, FA_ERR_PARAM_INVALID or
 * FA_ERR_UNSUPPORTED.  On error *plan is set to NULL.  No device work.
 */
fa_status fa_fwd_get_workspace_size(
    const fa_tensor* query, const fa_tensor* query_rope, const fa_tensor* key,
    const fa_tensor* key_rope, const fa_tensor* value, const fa_tensor* real_shift,
    const fa_tensor* atten_mask, const fa_tensor* sink, const fa_tensor* cu_seqlens_q,
    const fa_tensor* cu_seqlens_kv, const int64_t* q_start_idx, const int64_t* kv_start_idx,
    double scale_value, double keep_prob, int64_t pre_tokens,
    int64_t next_tokens, int64_t head_num, const char* input_layout, int64_t inner_precise,
    int64_t sparse_mode, int32_t causal, const char* softmax_out_layout,
    const fa_tensor* softmax_max, const fa_tensor* softmax_sum, const fa_tensor* attention_out,
    uint64_t* workspace_size, fa_plan** plan);

/*
 * Phase 2: enqueue the forward on `stream` (a hipStream_t; NULL = the null
 * stream).  Asynchronous: the caller synchronises.  `workspace` is a device
 * buffer of at least the size phase 1 reported (may be NULL when that size is
 * 0); the library uses it as scratch and it must not be in use by another
 * call on an overlapping stream.  Passage: V5 page, the second-phase call
 * (workspace, workspaceSize, executor, stream).
 *
 * Returns FA_OK, FA_ERR_PARAM_NULLPTR (plan NULL), FA_ERR_WORKSPACE or
 * FA_ERR_RUNTIME.  The plan is not consumed (see fa_plan_destroy): it may be
 * executed again, with the same or another workspace of sufficient size.
 */
fa_status fa_fwd(void* workspace, uint64_t workspace_size, const fa_plan* plan, void* stream);

/*
 * Phase 2 for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same work as
 * fa_fwd, with the library's own device scratch array (one per GPU, of
 * FA_NOALLOC_SCRATCH_BYTES, held until the process ends) in place of the
 * caller's workspace.  It allocates and frees nothing.  The array's device
 * address is looked up once per device on that device's first call.
 *
 * Every call on one GPU shares that GPU's array: calls whose device work may
 * overlap (on different streams, or on one stream from several threads
 * without ordering) race on it and must not be issued.  Nothing in the
 * array needs to start at zero; it keeps the last call's contents.
 *
 * Returns FA_OK, FA_ERR_PARAM_NULLPTR (plan NULL), FA_ERR_UNSUPPORTED (the
 * plan's workspace size, from phase 1, is above FA_NOALLOC_SCRATCH_BYTES) or
 * FA_ERR_RUNTIME.
 */
#define FA_NOALLOC_SCRATCH_BYTES (32ull << 20)
fa_status fa_fwd_noalloc(const fa_plan* plan, void* stream);

/*
 * Merge the results of one query chunk computed against several key chunks
 * (an outer split along the key sequence: one fa_fwd call per chunk with its
 * kv_start_idx, the sink given to one call only) into the result over all
 * keys.  With m_c, l_c the statistics of part c and O_c its output:
 *     m = max_c m_c,  w_c = e^(m_c - m) l_c,  l = sum_c w_c,
 *     O = sum_c w_c O_c / l
 * (from the definitions of softmaxMax / softmaxSum in the sink equations of
 * the V5 page, 功能说明 -> 计算公式).  Parts with m_c = -inf weigh nothing;
 * rows empty in every part get O = 0, m = -inf, l = 0.
 *
 *   n_parts             1..16.
 *   part_out            host array of n_parts descriptors, each shaped like
 *                       attention_out (same dtype, layout and sizes).
 *   part_max, part_sum  host arrays of n_parts F32 statistics descriptors in
 *                       the forward's statistics layout (required).
 *   input_layout, head_num, softmax_out_layout  as for phase 1.
 *   attention_out       merged output (F32, F16 or BF16).  It may be one of
 *                       the parts only if every part is read before it is
 *                       written: each row is read and written by one
 *                       wavefront, so aliasing a part row-for-row is safe.
 *   softmax_max, softmax_sum  optional merged statistics (NULL = not written).
 *   stream              hipStream_t; asynchronous, no workspace.
 * Returns FA_OK, FA_ERR_PARAM_NULLPTR, FA_ERR_PARAM_INVALID,
 * FA_ERR_UNSUPPORTED or FA_ERR_RUNTIME.
 */
fa_status fa_fwd_merge(int32_t n_parts, const fa_tensor* part_out, const fa_tensor* part_max,
                       const fa_tensor* part_sum, const char* input_layout, int64_t head_num,
                       const char* softmax_out_layout, const fa_tensor* attention_out,
                       const fa_tensor* softmax_max, const fa_tensor* softmax_sum, void* stream);

/* Release a plan from phase 1.  NULL is ignored.  Passage: V5 page, 调用示例,
 * which calls the second phase once and then releases the tensors and the
 * device memory but never the executor; the pages do not say whether the
 * second phase consumes it.  Here phase 2 does not: a plan may be executed
 * any number of times (repeated launches on fixed buffers), and the caller
 * releases it with this call when done.  A plan holds host memory only. */
void fa_plan_destroy(fa_plan* plan);

/* Text of the chosen kernel, tile and grid, e.g. for logs.  Writes at most
 * `len` bytes including the terminating NUL into `buf`; returns the length
 * the full text needs (excluding NUL), or -1 if plan or buf is NULL. */
int32_t fa_plan_describe(const fa_plan* plan, char* buf, size_t len);

/* Measurement utility (not part of the forward): enqueue on `stream` one
 * wavefront that idles for `microseconds` (1..1000000) of the GPU's constant
 * 100 MHz counter and writes to `device_out` (device memory, two uint64) the
 * shader-clock cycles and the 100 MHz ticks that passed, so that their ratio
 * is the shader clock while other work runs beside it.  Returns FA_OK,
 * FA_ERR_PARAM_NULLPTR, FA_ERR_UNSUPPORTED or FA_ERR_RUNTIME. */
fa_status fa_clock_probe(uint32_t microseconds, unsigned long long* device_out, void* stream);

/* Reason for the last non-zero status returned on the calling thread
 * (static, thread-local storage; never NULL). */
const char* fa_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_FWD_H */
