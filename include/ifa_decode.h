/*
 * ifa_decode.h — C ABI of the MI355X (gfx950) incremental decode-attention
 * library: paged split-KV decode attention, its combine step, and the
 * pairwise update of two attention results.
 *
 * What is computed (per batch b and query head h, query sequence length 1):
 *
 *   out[b,h] = sum_j e^(s_j - m) V_j / (sum_j e^(s_j - m) + e^(sink_h - m))
 *   s_j      = scale_value * q[b,h] . K_j,   j < actual_seq_lengths[b]
 *   m        = max(sink_h, max_j s_j)
 *   lse[b,h] = m + ln(sum_j e^(s_j - m) + e^(sink_h - m))
 *
 * Sources (page title, section):
 *   aclnnIncreFlashAttentionV3, "Function": Softmax(Q K^T / sqrt(d)) V for a
 *     query whose S axis is 1, per-batch actual KV lengths; "Function
 *     Prototype": the two-phase call (workspace size first, then launch on a
 *     stream); "Parameters": numHeads, numKeyValueHeads (0 = numHeads),
 *     scaleValue, blockSize, blocktable, antiquantScale/antiquantOffset;
 *     "Constraints": page attention scenario and the KV layout
 *     (blocknum, KV_N, blocksize, D); "Return Value": status codes.
 *   aclnnFlashAttentionScoreV4, "计算公式": learnable sink term.
 *   aclnnRingAttentionUpdate, "功能说明": update of an attention output from
 *     two (attn_out, softmax_max, softmax_sum) results.
 *   FusedInferAttentionScore blog (lpqz.cn): softmaxLse output, empty-tensor
 *     semantics.
 *
 * Conventions that the pages leave open, fixed here:
 *   - GQA: query head h reads KV head h / (num_heads / num_key_value_heads).
 *   - antiquant (int8 K/V): x_hat = (x + offset[i][g][d]) * scale[i][g][d],
 *     i = 0 for K, 1 for V, per KV head g and channel d, fp32 parameters.
 *   - the sink is a logit in the units of the scaled score s_j.
 *   - lse is a natural-log log-sum-exp and includes the sink term.
 *   - a sequence of length 0 gives out = 0 and lse = -inf (lse = sink_h with
 *     a sink).
 *   - RingAttentionUpdate is applied in its sum-weighted form:
 *       M = max(pm, cm); wp = ps e^(pm-M); wc = cs e^(cm-M) (0 when the max
 *       is -inf); sum = wp + wc; out = (wp po + wc co) / sum (0 when sum=0).
 *     With both sums equal to 1 this is the printed formula.
 *
 * Memory: the library never allocates and never synchronises.  Every pointer
 * is a device pointer owned by the caller unless stated otherwise, and must
 * stay valid until the work queued on `stream` has finished.  Calls are
 * asynchronous on `stream`.  Results are deterministic: split boundaries and
 * the merge order depend only on the arguments and the lengths.
 *
 * Errors: every entry point returns an ifa_status; no C++ exception crosses
 * the ABI.  On error nothing has been queued.  ifa_last_error() returns a
 * description of the most recent error on the calling thread.
 */
#ifndef IFA_DECODE_H
#define IFA_DECODE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes, mirroring the aclnn return codes of the pages
 * (aclnnIncreFlashAttentionV3 "Return Value"; aclnnMlaPrologV3WeightNz
 * "Return Value" for the tiling error). */
typedef enum {
  IFA_OK = 0,
  IFA_ERR_PARAM_NULLPTR = 161001, /* a required pointer is NULL */
  IFA_ERR_PARAM_INVALID = 161002, /* dtype, layout, shape or constraint */
  IFA_ERR_RUNTIME = 361001,       /* a HIP runtime call or launch failed */
  IFA_ERR_PLAN = 561002           /* workspace too small / no valid plan */
} ifa_status;

typedef enum { IFA_F32 = 0, IFA_F16 = 1, IFA_BF16 = 2, IFA_I8 = 3 } ifa_dtype;

typedef enum {
  /* contiguous, padded: (B, N_kv, s_cap, D); token j of batch b, KV head g
   * at ((b * N_kv + g) * s_cap + j) * D */
  IFA_KV_BNSD = 0,
  /* paged pool (num_blocks, N_kv, block_size, D): token j of batch b, KV
   * head g in block blk = block_table[b * max_blocks_per_seq + j / block_size]
   * at ((blk * N_kv + g) * block_size + j % block_size) * D */
  IFA_KV_PAGED = 1,
  /* paged pool (num_blocks, block_size, H), H = N_kv * D, the other layout of
   * aclnnIncreFlashAttentionV3 "Constraints" (page attention scenario): head
   * g holds columns g * D .. g * D + D - 1 of H, so token j of batch b, KV
   * head g is at ((blk * block_size + j % block_size) * N_kv + g) * D */
  IFA_KV_PAGED_BSH = 2,
  /* contiguous, padded (B, s_cap, H), the BSH / BSND key and value layouts
   * of the same page's "Parameters": ((b * s_cap + j) * N_kv + g) * D */
  IFA_KV_BSND = 3
} ifa_kv_layout;

/* Antiquant parameter shapes (aclnnIncreFlashAttentionV3 "Constraints" on
 * antiquantScale and antiquantOffset): per channel (2, N_kv, qk_dim), or per
 * tensor (2); index 0 applies to K, 1 to V.  Per token (the
 * FusedInferAttentionScore blog's antiquantMode 1 per-token and 3 per-token
 * with per-head, whose shapes the pages do not print): fp32 (2, B, S), or
 * (2, B, N_kv, S) per token and KV head, one (scale, offset) pair per logical
 * token position j < S of sequence b, applied to every channel of that
 * token; S is s_cap for the contiguous layouts and max_blocks_per_seq *
 * block_size for the paged ones.  Per-token modes need qk_dim 128. */
typedef enum {
  IFA_ANTIQUANT_PER_CHANNEL = 0,
  IFA_ANTIQUANT_PER_TENSOR = 1,
  IFA_ANTIQUANT_PER_TOKEN = 2,
  IFA_ANTIQUANT_PER_TOKEN_HEAD = 3
} ifa_antiquant_mode;

/* Masks of a multi-token decode (the sparseMode values of the
 * FusedInferAttentionScore pages).  With S_q query tokens per sequence of
 * actual length L, query i is the token at position L - S_q + i:
 *   IFA_MASK_NONE   every query attends to all L tokens;
 *   IFA_MASK_CAUSAL rightDownCausal: query i attends to tokens j <= L - S_q + i;
 *   IFA_MASK_TREE   treeMask of speculative decoding: every query attends to
 *                   the tokens before the last S_q, and to the last-S_q token k
 *                   iff tree_mask[b][i][k] == 0 (1 removes it).
 * A query left with no token gives attention_out 0 and softmax_lse -inf. */
typedef enum { IFA_MASK_NONE = 0, IFA_MASK_CAUSAL = 3, IFA_MASK_TREE = 9 } ifa_sparse_mode;

/* Arguments of one decode call.  Element strides are implied by the shapes;
 * every tensor is dense and row-major as described. */
typedef struct {
  const void* query;          /* (B, N_q, qk_dim), q_dtype */
  const void* key_cache;      /* layout per kv_layout, row length qk_dim, kv_dtype */
  const void* value_cache;    /* row length v_dim; MAY EQUAL key_cache, then V is
                                 the first v_dim channels of each key row (MLA) */
  const int32_t* block_table; /* (B, max_blocks_per_seq), the paged layouts only */
  const int64_t* actual_seq_lengths; /* (B), device; values in [0, s_cap] */
  const float* learnable_sink;       /* (N_q) or NULL */
  const float* antiquant_scale;      /* fp32, shape per antiquant_mode; required iff kv_dtype is IFA_I8 */
  const float* antiquant_offset;     /* fp32, the shape of antiquant_scale; required iff kv_dtype is IFA_I8 */
  void* attention_out;               /* (B, N_q, v_dim), out_dtype */
  float* softmax_lse;                /* (B, N_q) fp32, or NULL */
  int64_t batch;                     /* B >= 0; B == 0 is a no-op */
  int64_t num_heads;                 /* N_q, 1..256 */
  int64_t num_key_value_heads;       /* N_kv; 0 means N_q; N_q % N_kv == 0 */
  int64_t qk_dim;                    /* 64, 128, or 576 (MLA) */
  int64_t v_dim;                     /* == qk_dim, or 512 with qk_dim 576 (MLA) */
  int64_t block_size;                /* paged: multiple of 16 (32 for int8), 16..1024 */
  int64_t max_blocks_per_seq;        /* paged: second dim of block_table */
  int64_t num_blocks;                /* paged: pool size; block ids are clamped to it
                                        (ifa_decode_check_inputs reports ids outside it) */
  int64_t s_cap;                     /* contiguous: padded length; lengths are clamped to it
                                        (ifa_decode_check_inputs reports lengths outside it) */
  double scale_value;                /* usually 1/sqrt(d) */
  int32_t q_dtype;                   /* IFA_F32 / IFA_F16 / IFA_BF16 */
  int32_t kv_dtype;                  /* == q_dtype, or IFA_I8 */
  int32_t out_dtype;                 /* IFA_F32 / IFA_F16 / IFA_BF16 */
  int32_t kv_layout;                 /* ifa_kv_layout */
  int32_t num_splits;                /* KV-axis splits per sequence, 1..256; 0 = auto */
  int32_t antiquant_mode;            /* ifa_antiquant_mode; 0 unless kv_dtype is IFA_I8 */
  /* multi-token decode (speculative verification), GQA shapes only: S_q =
   * q_seq_len query tokens per sequence (0 means 1; at most 16).  Then query
   * is (B, S_q, N_q, qk_dim), attention_out (B, S_q, N_q, v_dim) and
   * softmax_lse (B, S_q, N_q); with S_q == 1 these are the shapes above. */
  int64_t q_seq_len;
  const uint8_t* tree_mask;          /* (B, S_q, S_q) device, IFA_MASK_TREE only */
  int32_t sparse_mode;               /* ifa_sparse_mode */
  int32_t reserved;                  /* must be 0 */
} ifa_decode_args;

/* Phase 1 (aclnnIncreFlashAttentionV3GetWorkspaceSize): validate `args` and
 * return in *workspace_bytes the device scratch the decode needs for its
 * split partials.  Pure host code; never touches device memory.  Device
 * pointers are checked for NULL only. */
ifa_status ifa_decode_workspace_size(const ifa_decode_args* args, size_t* workspace_bytes);

/* The number of KV-axis splits per sequence that a call with `args` uses
 * (args->num_splits, or the automatic choice when it is 0).  Split i of a
 * sequence of length L covers tokens [i*c, min(L, (i+1)*c)) with
 * c = 16 * ceil(ceil(L / n) / 16); splits past the end are empty.
 * With the balanced split (ifa_decode_split_mode) it is instead the number
 * of runs n the whole batch is cut into. */
ifa_status ifa_decode_num_splits(const ifa_decode_args* args, int32_t* num_splits);

/* Whether a call with `args` splits per sequence (*balanced = 0) or
 * balanced (1).  The balanced split is the automatic choice (num_splits 0)
 * for batch <= 256 of the MLA shape (when a run spans at most 1022 cache
 * blocks) and of the GQA shapes that run on the matrix cores (head dim 128
 * with 16-bit or int8 K/V).  Every sequence with L > 0 tokens is cut into
 * t = ceil(L / 32) tiles (the last one ragged) and weighs P + t units: P for
 * starting a piece on it (7 on the MLA shape, 8 on the GQA shapes), then one
 * per tile.  The V units of the batch, sequence after sequence, are cut into
 * R = min(n, V) runs, run r the units [floor(r V / R), floor((r + 1) V / R))
 * (n = ifa_decode_num_splits); a run takes the tiles whose units it holds.
 * Each run is one workgroup per (KV head, group of query rows), so the work
 * per compute unit is about the same whatever the mix of lengths; a run's
 * piece of sequence b is one partial, in slot r + b. */
ifa_status ifa_decode_split_mode(const ifa_decode_args* args, int32_t* balanced);

/* Phase 2 (aclnnIncreFlashAttentionV3): split-KV decode followed by the
 * combine, queued on `stream`.  `workspace` must hold at least the bytes
 * phase 1 returned (IFA_ERR_PLAN otherwise); it may be NULL when that size
 * is 0.  Writes attention_out and, when non-NULL, softmax_lse. */
ifa_status ifa_decode(const ifa_decode_args* args, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/* First half of ifa_decode: computes, for every (batch, query head, split),
 * the partial triple over the split's tokens and stores it in `workspace`:
 *   attn_out    fp32 [B][N_q][n][v_dim]   softmax-normalised over the split
 *   softmax_max fp32 [B][N_q][n]          max of the scaled logits (natural units)
 *   softmax_sum fp32 [B][N_q][n]          sum of e^(s_j - softmax_max)
 * in that order, each array starting at a 256-byte aligned offset; on the
 * MLA shape (qk_dim 576, v_dim 512, one KV head) attn_out is fp16, rounded
 * to nearest even (max and sum stay fp32): a normalised partial is a convex
 * combination of V rows, so it is exact to fp16 rounding while |V| stays
 * below 65504 (larger V overflows the partial)
 * (n = ifa_decode_num_splits).  Empty splits are not written; the sink is not
 * applied here.  When batch <= 256 a fourth array follows, int32 pairs [B]:
 * (sequence, clamped length) in descending length order (ties by index).
 * On the int8-KV path a small planning kernel writes it first and the
 * split-KV kernel dispatches its work by it (longest sequences first); the
 * other paths rank the lengths inside the split-KV kernel and leave it
 * unused.
 * The balanced split lays the partials out by slot instead: attn_out fp32
 * (fp16 on the MLA shape) [n + B][S_q][N_q][v_dim], softmax_max and
 * softmax_sum fp32 [n + B][S_q][N_q]
 * (S_q = query tokens per sequence), and the
 * fourth array holds, for each sequence with at least one token, the int32
 * pair (first slot, number of slots) of its pieces, in token order. */
ifa_status ifa_decode_splitkv(const ifa_decode_args* args, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/* Size of the fixed device array that ifa_decode_noalloc keeps its split
 * partials in (per device, held until the process ends): 128 MiB. */
#define IFA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): ifa_decode
 * with no workspace argument.  The split partials go to a fixed array of
 * IFA_NOALLOC_SCRATCH_BYTES that the library holds on each device it runs
 * on; the call allocates nothing and computes exactly what ifa_decode
 * computes.  The caller still passes every input and output in `args`, on the
 * device current at the call (the first call on a device takes the array's
 * address with that device current).  A call whose partials need more than
 * the array (ifa_decode_workspace_size) fails with IFA_ERR_PLAN before
 * anything is queued.  All calls on one device share the array: calls that
 * overlap on one device (different streams, or unordered threads) race. */
ifa_status ifa_decode_noalloc(const ifa_decode_args* args, hipStream_t stream);

/* ifa_decode_splitkv for measurement: the same work, launched so that the
 * runtime records `start` and `stop` (events the caller created on this
 * device with timing enabled) at the split-KV kernel's own start and end
 * (hipExtLaunchKernel), which an event recorded around the call on the stream
 * cannot do as tightly.  IFA_ERR_PARAM_NULLPTR if either event is NULL;
 * with batch 0 nothing is launched and the events are not recorded. */
ifa_status ifa_decode_splitkv_timed(const ifa_decode_args* args, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream, hipEvent_t start, hipEvent_t stop);

/* Second half of ifa_decode: merges the non-empty split partials of each
 * (batch, query head) in split order with the RingAttentionUpdate rule, folds
 * in the learnable sink as one more partial (attn_out 0, max sink_h, sum 1),
 * and writes attention_out (cast with round-to-nearest-even) and
 * softmax_lse. */
ifa_status ifa_decode_combine(const ifa_decode_args* args, const void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* aclnnRingAttentionUpdate: updates one attention result with another.
 *   prev_attn_out, cur_attn_out, attn_out: (rows, head_dim), dtype
 *     IFA_F32 / IFA_F16 / IFA_BF16 (all three the same dtype);
 *   *_softmax_max, *_softmax_sum: fp32 (rows, stat_stride); stat_stride is
 *     1, or 8 for the pages' layout whose last dimension repeats each value
 *     8 times (only element 0 of each row is read; all stat_stride elements
 *     are written).
 * Outputs may alias the prev or cur inputs (in-place accumulation).  A max of
 * -inf with a sum of 0 marks an empty result.  rows == 0 is a no-op. */
ifa_status attn_update(const void* prev_attn_out, const float* prev_softmax_max,
                       const float* prev_softmax_sum, const void* cur_attn_out,
                       const float* cur_softmax_max, const float* cur_softmax_sum,
                       void* attn_out, float* softmax_max_out, float* softmax_sum_out,
                       int64_t rows, int64_t head_dim, int32_t dtype, int32_t stat_stride,
                       hipStream_t stream);

/* Paged KV-cache write, the step before a decode step
 * (aclnnMlaPrologV3WeightNz "Parameters": kvCacheRef / krCacheRef updated in
 * place at cacheIndexOptional, CacheMode PA_BSND).  For every token t and KV
 * head g, the d elements src[t][g][0 .. d-1] are copied unchanged into
 * elements col_offset .. col_offset + d - 1 of the cache row of slot
 * s = slot_index[t], which is position s % block_size of block
 * s / block_size:
 *   layout IFA_KV_PAGED_BSH: cache (num_blocks, block_size, N_kv, row_elems)
 *   layout IFA_KV_PAGED:     cache (num_blocks, N_kv, block_size, row_elems)
 * (the MLA row [latent 512 | rope 64] takes two calls, col_offset 0 and 512).
 *   src        (tokens, num_kv_heads, d), device, element type `dtype`
 *   slot_index (tokens) int64, device; a slot outside
 *              [0, num_blocks * block_size) is skipped
 *   cache      device, element type `dtype`, written in place
 * d, col_offset and row_elems must each span a multiple of 16 bytes, and
 * src and cache must be 16-byte aligned (IFA_ERR_PARAM_INVALID otherwise).
 * Two tokens naming the same slot leave one of the two rows there.
 * tokens == 0 is a no-op.  Asynchronous on `stream`. */
ifa_status ifa_kv_cache_write(const void* src, const int64_t* slot_index, void* cache, int64_t tokens,
                              int64_t num_kv_heads, int64_t d, int64_t row_elems, int64_t col_offset,
                              int64_t num_blocks, int64_t block_size, int32_t layout, int32_t dtype,
                              hipStream_t stream);

/* Block count of a paged pool (aclnnMlaPrologV3WeightNz "Constraints",
 * BlockNum row): sum over b of ceil(lengths[b] / block_size).  Host pointer;
 * returns -1 for a NULL pointer, a negative batch or length, or a block_size
 * below 1. */
int64_t ifa_paged_block_count(const int64_t* lengths, int64_t batch, int64_t block_size);

/* Reports the arguments that ifa_decode would clamp rather than follow.  The
 * decode clamps a length to [0, S] (S = s_cap, or max_blocks_per_seq *
 * block_size for the paged layouts) and a block id to [0, num_blocks), so a
 * corrupt argument never takes it outside its buffers but silently changes
 * the result.  This call queues, on `stream`, one small kernel that reads the
 * lengths and every block-table entry the decode would read (entries
 * 0 .. ceil(clamped length / block_size) - 1 of each row) and writes to
 * `flags` (one device int32, overwritten) the OR of
 *   IFA_CHECK_BAD_LENGTH (1): a length outside [0, S];
 *   IFA_CHECK_BAD_BLOCK  (2): a block-table entry outside [0, num_blocks).
 * 0 means the call's lengths and table are in range.  The other arguments
 * are validated as by ifa_decode_workspace_size; no workspace is needed.
 * Asynchronous: read `flags` after the stream's work has finished. */
#define IFA_CHECK_BAD_LENGTH 1
#define IFA_CHECK_BAD_BLOCK 2
ifa_status ifa_decode_check_inputs(const ifa_decode_args* args, int32_t* flags, hipStream_t stream);

/* Measurement helper: the HBM read rate of this device, for setting the
 * decode's achieved bandwidth against a ceiling measured in the same run.
 * Reads every 16-byte chunk of `buf` (device, 16-byte aligned, `bytes` a
 * multiple of 16) once with non-temporal loads spread over `workgroups`
 * workgroups of 256 lanes, and writes one 32-bit word per workgroup to `out`
 * (device, `workgroups` words; the XOR of what the workgroup read, which
 * keeps the loads live).  Asynchronous on `stream`; bytes == 0 is a no-op.
 * IFA_ERR_PARAM_INVALID for workgroups outside [1, 2^20] or misaligned
 * sizes, IFA_ERR_PARAM_NULLPTR for a NULL pointer. */
ifa_status ifa_read_bandwidth_probe(const void* buf, size_t bytes, uint32_t* out, int32_t workgroups,
                                    hipStream_t stream);

/* Description of the last error on the calling thread ("" if none).  The
 * string is owned by the library and valid until the next call on the
 * thread. */
const char* ifa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* IFA_DECODE_H */
