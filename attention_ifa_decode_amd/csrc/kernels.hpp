// Launch descriptors shared by the host library and the kernel files.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ifa {

// Split-KV decode of the GQA shapes: the MFMA kernel (head dim 128, 16-bit or
// int8 K/V) and the VALU kernel (f32 K/V, head dim 64) take the same launch.
struct GqaLaunch {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* block_table;
  const int64_t* seq_lens;
  const float* aq_scale;   // (2, n_kv, D) or (2), or null
  const float* aq_offset;  // the shape of aq_scale
  // entry (i, g, d) of the parameters, i = 0 for K and 1 for V:
  // i * aq_stride_kv + g * aq_stride_g + d * aq_stride_d
  int aq_stride_kv, aq_stride_g, aq_stride_d;
  // per-token antiquant (MFMA path): entry (i, b, g, token j) of
  // (2, B, S) or (2, B, N_kv, S) parameters at
  // i * aq_tok_stride_kv + b * aq_tok_stride_b + g * aq_tok_stride_g + j
  bool aq_token;
  int64_t aq_tok_stride_kv, aq_tok_stride_b, aq_tok_stride_g;
  float* ws_o;             // [B][q_seq][n_q][n_split][D] (balanced split: by slot, below)
  float* ws_m;             // [B][q_seq][n_q][n_split]
  float* ws_l;             // [B][q_seq][n_q][n_split]
  int batch, n_q, n_kv, group, heads_per_wg, n_split;
  // multi-token decode: q_seq query tokens per sequence; the rows_kv =
  // q_seq * group query rows of a KV head (query token major) are split into
  // workgroups of heads_per_wg rows
  int q_seq, rows_kv;
  int mask_mode;               // 0 none, 3 rightDownCausal, 9 tree
  const uint8_t* tree_mask;    // (B, q_seq, q_seq), 1 removes a draft token
  int64_t s_cap;           // lengths are clamped to this
  int block_size, max_blocks, num_blocks;
  uint32_t bs_magic, bs_shift;  // n / block_size == (umulhi(n, magic) + n) >> shift
  float scale_log2;        // scale * log2(e)
  int q_dtype, kv_dtype, head_dim;
  bool paged;
  bool token_major;        // (blocks, block_size, N_kv, D) / (B, s_cap, N_kv, D) instead of head-major
  const int2* plan;        // [batch] (sequence, clamped length) in longest-first order, or null
  bool longest_first;      // without a plan: each workgroup ranks the lengths itself
  // Balanced split of the MFMA kernel (batch <= kLongestFirstMaxBatch): the
  // batch's 32-token tiles, sequence after sequence, each sequence's first
  // one weighted kGqaPieceCost more, are cut into n_split runs of equal
  // weight, the same runs for every KV head; run r's piece of sequence b
  // writes partial slot r + b ([slot][q_seq][n_q] statistics,
  // [slot][q_seq][n_q][D] outputs), and seg_desc[b] = (first slot, slot count).
  bool balanced;
  int2* seg_desc;
};

// MLA-shaped decode: all query heads share one latent KV head (MFMA path).
struct MlaLaunch {
  const void* q;           // (B, n_q, qk_dim) bf16
  const void* kv;          // pool (num_blocks, 1, block_size, qk_dim) bf16; V = first v_dim channels
  const int32_t* block_table;
  const int64_t* seq_lens;
  // partial outputs in fp16 (statistics in fp32): a normalised partial is a
  // convex combination of V rows, so it stays within fp16's range when V does
  _Float16* ws_o;
  float* ws_m;
  float* ws_l;
  int batch, n_q, n_split;
  int64_t s_cap;
  int block_size, max_blocks, num_blocks;
  uint32_t bs_magic, bs_shift;
  float scale_log2;
  int qk_dim, v_dim;
  bool paged;
  bool longest_first;      // each workgroup ranks the lengths and takes its rank's sequence
  // Balanced split (batch <= kLongestFirstMaxBatch): the batch's 32-token
  // tiles, sequence after sequence, each sequence's first one weighted
  // kMlaPieceCost more, are cut into n_split runs of equal weight; run r's
  // piece of sequence b writes partial slot r + b ([slot][n_q] statistics,
  // [slot][n_q][v_dim] outputs), and seg_desc[b] = (first slot, slot count).
  bool balanced;
  int2* seg_desc;
};

struct CombineLaunch {
  const void* ws_o;   // partial outputs: fp32, or fp16 when o_f16 (the MLA path)
  bool o_f16;
  const float* ws_m;
  const float* ws_l;
  const int64_t* seq_lens;
  const float* sink;  // (n_q) or null
  void* out;          // (batch, n_q, v_dim)
  float* lse;         // (batch, n_q) or null
  int batch, n_q, n_split, v_dim, out_dtype;  // batch counts (sequence, query token) pairs
  int q_seq;          // query tokens per sequence: row r belongs to sequence r / n_q / q_seq
  int64_t s_cap;
  // balanced split (MLA and GQA MFMA paths): sequence b's partials are slots
  // seg_desc[b].x .. + seg_desc[b].y - 1 of a [slot][q_seq][n_q] layout;
  // null for the per-sequence [row][n_split] layout
  const int2* seg_desc;
};

struct UpdateLaunch {
  const void* prev_out;
  const float* prev_max;
  const float* prev_sum;
  const void* cur_out;
  const float* cur_max;
  const float* cur_sum;
  void* out;
  float* max_out;
  float* sum_out;
  int64_t rows;
  int head_dim, dtype, stat_stride;
};

// Token span of split `split` out of `n_split` for a sequence of length L:
// [split * c, min(L, (split + 1) * c)), c = 16 * ceil(ceil(L / n) / 16).
__host__ __device__ inline int64_t split_chunk(int64_t L, int n_split) {
  int64_t per = (L + n_split - 1) / n_split;
  return (per + 15) & ~int64_t(15);
}

// Magic-number division by a runtime divisor d in [1, 2^31): for n < 2^31,
// n / d == (umulhi(n, magic) + n) >> shift  (Granlund-Montgomery).
inline void make_divisor(uint32_t d, uint32_t* magic, uint32_t* shift) {
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  *shift = s;
  *magic = (uint32_t)((((1ull << s) - d) << 32) / d + 1);
  if (d == 1) *magic = 0;  // (0 + n) >> 0
}

__device__ __forceinline__ uint32_t fast_div(uint32_t n, uint32_t magic, uint32_t shift) {
  return (__umulhi(n, magic) + n) >> shift;
}

// Largest batch for which the workgroups rank sequences by length on the device.
constexpr int kLongestFirstMaxBatch = 256;

// Most block-table entries one split of the MLA path may touch (staged in LDS).
constexpr int kMlaMaxTableSlice = 1024;
// Balanced split of the MLA path: the cost, in tiles, charged to a sequence
// for the start of a piece on it.
constexpr int kMlaPieceCost = 7;
// The same for the balanced split of the GQA MFMA kernel (one wave per
// workgroup: Q, block-table slice and first tile are three dependent memory
// round trips, each a few microseconds under load, against about a
// microsecond per streamed tile).
constexpr int kGqaPieceCost = 8;

// Optional events that a launch records around the kernel itself
// (hipExtLaunchKernel), for measuring the kernel's own duration.
struct LaunchEvents {
  hipEvent_t start, stop;
};

template <typename K, typename... A>
inline void launch_kernel(K kernel, dim3 grid, dim3 block, hipStream_t stream, const LaunchEvents* ev, A... args) {
  if (ev)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, ev->start, ev->stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, args...);
}

hipError_t launch_gqa_splitkv(const GqaLaunch& p, hipStream_t stream, const LaunchEvents* ev = nullptr);
// GQA decode on the matrix cores (any number of query tokens): one wave per
// (sequence, KV head, group of 16 or 32 query rows, split); 16-bit K/V, or
// int8 K/V with per-channel, per-tensor or per-token antiquant, head dim 128.
bool gqa_mfma_supported(int q_dtype, int kv_dtype, int head_dim);
hipError_t launch_gqa_mfma(const GqaLaunch& p, hipStream_t stream, const LaunchEvents* ev = nullptr);
hipError_t launch_mla_splitkv(const MlaLaunch& p, hipStream_t stream, const LaunchEvents* ev = nullptr);
hipError_t launch_combine(const CombineLaunch& p, hipStream_t stream);
// One workgroup: plan[r] = (sequence, clamped length) of the r-th longest
// sequence, for the longest-first dispatch of the split-KV kernels.
hipError_t launch_plan(const int64_t* seq_lens, int batch, int64_t cap, int2* plan, hipStream_t stream);
hipError_t launch_update(const UpdateLaunch& p, hipStream_t stream);
// Input check: bit kCheckBadLength if a length lies outside [0, s_cap], bit
// kCheckBadBlock if a block-table entry the call reads lies outside
// [0, num_blocks); one int32 word to flags.
constexpr int32_t kCheckBadLength = 1, kCheckBadBlock = 2;
struct CheckLaunch {
  const int64_t* seq_lens;
  const int32_t* block_table;  // null for the contiguous layouts
  int32_t* flags;
  int64_t batch, s_cap, block_size, max_blocks, num_blocks;
};
hipError_t launch_check(const CheckLaunch& p, hipStream_t stream);

// Read-stream probe: reads bytes / 16 chunks of buf once, writes one word per
// workgroup to out.
hipError_t launch_read_probe(const void* buf, uint64_t bytes, uint32_t* out, int workgroups, hipStream_t stream);

// Paged KV-cache write: source rows (tokens, n_kv, row_chunks * 16 bytes) to
// the pool rows of their slots, at byte col_bytes of each row_bytes-long row.
struct CacheWriteLaunch {
  const void* src;
  const int64_t* slot_index;  // (tokens)
  void* cache;
  int64_t tokens, n_kv, row_chunks, row_bytes, col_bytes, num_blocks, block_size;
  bool token_major;           // (blocks, block_size, n_kv, W) rather than (blocks, n_kv, block_size, W)
};
hipError_t launch_cache_write(const CacheWriteLaunch& p, hipStream_t stream);

// Which (q dtype, kv dtype, head dim, heads per workgroup) the VALU path has
// kernels for.
bool gqa_supported(int q_dtype, int kv_dtype, int head_dim, int heads_per_wg);
int gqa_max_heads_per_wg(int kv_dtype, int head_dim);

// Query head counts the MLA (MFMA) path has kernels for: multiples of 32.
bool mla_supported(int n_q);

}  // namespace ifa
