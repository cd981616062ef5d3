// Host side of the C ABI: argument validation, split planning, workspace
// sizing and kernel launches.  No allocation, no synchronisation.
//
// The call shape follows the two-phase API of aclnnIncreFlashAttentionV3
// ("Function Prototype": GetWorkspaceSize validates and sizes, then the
// second call runs on a stream) and its checks follow "Constraints"
// (N <= 256, numHeads a multiple of numKeyValueHeads, page-attention blockSize
// alignment, blockTable with B rows) and "Return Value" (161001 null pointer,
// 161002 invalid parameter, 361001 runtime error).  561002 (tiling error,
// aclnnMlaPrologV3WeightNz "Return Value") reports an unusable workspace.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/ifa_decode.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_last_error;

ifa_status fail(ifa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

ifa_status ok() {
  g_last_error.clear();
  return IFA_OK;
}

constexpr int kTargetCUs = 256;       // MI355X compute units
constexpr int kMaxSplits = 256;
constexpr int64_t kMaxBatch = 65536;  // aclnnIncreFlashAttentionV3 Constraints: B <= 65536
constexpr int64_t kMaxHeads = 256;    // N <= 256

enum class Path { kGqa, kMla };

struct Plan {
  Path path;
  int64_t n_kv;
  int group;
  int heads_per_wg;  // query rows per workgroup (GQA)
  int q_seq;         // query tokens per sequence
  bool mfma;         // GQA rows on the matrix cores (multi-token decode)
  bool balanced;     // MLA: equal runs of the whole batch's tiles (n_split runs)
  int n_split;
  size_t off_o, off_m, off_l, off_plan, bytes;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool is_float_dtype(int32_t d) { return d == IFA_F32 || d == IFA_F16 || d == IFA_BF16; }

// Automatic split count of the GQA kernel.  Each workgroup pays a fixed
// start (three dependent memory round trips, about 12-15 us under load) and
// streams a single item, so fewer, longer items win until the GPU runs out
// of parallel work.  Measured on MI355X, whole-step time over split counts:
// bf16 / f16 shapes are fastest at about 256-512 workgroups in all (e.g. the
// padded fp16 B=16 decode: 27 us at 4 splits, 41 us at 16), int8 KV, which
// does more arithmetic per byte, at about 2048 (B=32, 16K tokens: 345 us at
// 4 splits, 434 us at 1).  A split also keeps at least ~1024 tokens of the
// longest sequence.
int auto_splits_gqa(const ifa_decode_args* a, int64_t n_kv, int rows_kv, int gh, int64_t max_len) {
  const int64_t per_split = a->batch * n_kv * (rows_kv / gh);  // workgroups per split index
  const int64_t target = a->kv_dtype == IFA_I8 ? 8LL * kTargetCUs : 2LL * kTargetCUs;
  int64_t n = (target + per_split - 1) / per_split;
  const int64_t by_len = (max_len + 1023) / 1024;
  if (n > by_len) n = by_len;
  if (n < 1) n = 1;
  if (n > 64) n = 64;
  return (int)n;
}

// One-wave workgroups of the MFMA path: about 2048 of them, each split at
// least 384 tokens long (measured over batch 1 to 64 and lengths 512 to 32768).
int auto_splits_mfma(const ifa_decode_args* a, int64_t n_kv, int rows_kv, int64_t max_len) {
  const int64_t per_split = a->batch * n_kv * ((rows_kv + 31) / 32);
  int64_t n = (8LL * kTargetCUs + per_split - 1) / per_split;
  const int64_t by_len = (max_len + 383) / 384;
  if (n > by_len) n = by_len;
  if (n < 1) n = 1;
  if (n > 128) n = 128;
  return (int)n;
}

// Balanced split of the GQA MFMA kernel: runs of the batch's 32-token tiles,
// the same runs for every KV head, one one-wave workgroup per (run, KV head,
// group of query rows).  The runs are sized to one round of resident
// workgroups (measured per-workgroup residency: 4 per CU with the 16-bit
// kernel's 32 KB of LDS, 8 per CU with the int8 kernel's 16 KB, where two
// waves per SIMD are the register limit): every run starts at once and they
// finish together, where a second round of equal runs would start in step
// and pay the start of a workgroup twice (2048 runs of 16-bit rows measured
// 2-25% slower than 1024).  Short runs cost little more than long ones: the
// runs start together, so their starts overlap, and small batches gain most
// from the full round (two sequences of about 2000 tokens: 15.5 us at 128
// runs, 26.3 us at 9, 21.1 us with the per-sequence split).  The only bound is
// one run per cost unit at the longest lengths; more runs would hold no work.
// The per-sequence split sizes its splits by each sequence's length, so with
// mixed lengths the longest splits (and the tail of the kernel) are about
// twice the mean; equal runs finish together.
int balanced_runs_gqa(const ifa_decode_args* a, int64_t n_kv, int rows_kv, int64_t max_len) {
  const int64_t per_run = n_kv * ((rows_kv + (rows_kv <= 16 ? 15 : 31)) / (rows_kv <= 16 ? 16 : 32));
  const int64_t resident = (a->kv_dtype == IFA_I8 ? 8LL : 4LL) * kTargetCUs;
  int64_t r = (resident + per_run - 1) / per_run;
  const int64_t units = a->batch * ((max_len + 31) / 32 + ifa::kGqaPieceCost);
  if (r > units) r = units;
  return (int)(r < 1 ? 1 : (r > kMaxSplits ? kMaxSplits : r));
}

// The automatic choice of the GQA MFMA kernel when the batch allows it (the
// plan region holds one (first slot, count) pair per sequence, batch <= 256)
// and the batch's cost units stay in 32 bits.  int8 K/V with more than 16
// query rows per KV head (32-column MFMAs) keeps the per-sequence split: its
// balanced kernel would not fit two waves per SIMD.
bool use_balanced_gqa(const ifa_decode_args* a, int rows_kv, int64_t max_len) {
  if (a->num_splits != 0 || a->batch > ifa::kLongestFirstMaxBatch) return false;
  if (a->kv_dtype == IFA_I8 && rows_kv > 16) return false;
  return a->batch * ((max_len + 31) / 32 + ifa::kGqaPieceCost) < (int64_t)1 << 31;
}

// Fewest splits for which one split of the longest sequence touches at most
// kMlaMaxTableSlice block-table entries (paged layout).
bool is_paged(int layout) { return layout == IFA_KV_PAGED || layout == IFA_KV_PAGED_BSH; }
// token-major layouts: consecutive tokens of one KV head are N_kv rows apart
bool is_token_major(int layout) { return layout == IFA_KV_PAGED_BSH || layout == IFA_KV_BSND; }

int64_t min_splits_mla(const ifa_decode_args* a, int64_t max_len) {
  if (!is_paged(a->kv_layout)) return 1;
  for (int64_t n = 1; n <= kMaxSplits; ++n)
    if (ifa::split_chunk(max_len, (int)n) <= (int64_t)(ifa::kMlaMaxTableSlice - 2) * a->block_size) return n;
  return kMaxSplits + 1;
}

// Balanced split of the MLA path: runs of the batch's 32-token tiles, one
// workgroup each, about one workgroup per compute unit whatever the number
// of head groups (each workgroup holds up to 128 heads), at most 256 (the
// combine's slots per sequence).
int balanced_runs(const ifa_decode_args* a) {
  const int64_t r = kTargetCUs * 128LL / a->num_heads;
  return (int)(r < 1 ? 1 : (r > kMaxSplits ? kMaxSplits : r));
}

// The automatic choice for the MLA shape when the batch allows it: the plan
// region holds one (first slot, count) pair per sequence (batch <= 256), tile
// counts stay in 32 bits, and a run spans at most kMlaMaxTableSlice - 2 cache
// blocks.  Measured on the MLA config (B 32, lengths 1K..32K): about 20 us per
// workgroup item goes to loading Q, filling the ring and writing 256 KB of
// partials, and 16 splits per sequence left CUs idle for about 25 us of the
// tail; equal runs pay the start once per piece and finish together (a
// run's extra pieces are paid for by its weight: kMlaPieceCost).
bool use_balanced_mla(const ifa_decode_args* a, int64_t max_len) {
  if (a->num_splits != 0 || a->batch > ifa::kLongestFirstMaxBatch) return false;
  const int64_t tiles = a->batch * ((max_len + 31) / 32 + ifa::kMlaPieceCost);
  if (tiles >= (int64_t)1 << 31) return false;
  const int64_t runs = balanced_runs(a);
  const int64_t run_tokens = 32 * ((tiles + runs - 1) / runs);
  return !is_paged(a->kv_layout) || run_tokens <= (int64_t)(ifa::kMlaMaxTableSlice - 2) * a->block_size;
}

int auto_splits_mla(const ifa_decode_args* a, int64_t max_len) {
  // one workgroup per compute unit at a time: about two items per CU, each
  // split at least 512 tokens long
  int64_t n = (2LL * kTargetCUs + a->batch - 1) / a->batch;
  const int64_t by_len = (max_len + 511) / 512;
  if (n > by_len) n = by_len;
  if (n < 1) n = 1;
  if (n > 64) n = 64;
  const int64_t lo = min_splits_mla(a, max_len);
  if (n < lo) n = lo;
  return (int)n;
}

ifa_status validate_and_plan(const ifa_decode_args* a, Plan* plan) {
  if (!a) return fail(IFA_ERR_PARAM_NULLPTR, "args is NULL");
  if (a->batch < 0 || a->batch > kMaxBatch)
    return fail(IFA_ERR_PARAM_INVALID, "batch %lld outside [0, %lld]", (long long)a->batch, (long long)kMaxBatch);
  if (a->num_heads < 1 || a->num_heads > kMaxHeads)
    return fail(IFA_ERR_PARAM_INVALID, "num_heads %lld outside [1, 256]", (long long)a->num_heads);
  if (a->num_key_value_heads < 0 || a->num_key_value_heads > a->num_heads)
    return fail(IFA_ERR_PARAM_INVALID, "num_key_value_heads %lld outside [0, num_heads]",
                (long long)a->num_key_value_heads);
  const int64_t n_kv = a->num_key_value_heads == 0 ? a->num_heads : a->num_key_value_heads;
  if (a->num_heads % n_kv)
    return fail(IFA_ERR_PARAM_INVALID, "num_heads %lld is not a multiple of num_key_value_heads %lld",
                (long long)a->num_heads, (long long)n_kv);
  if (!is_float_dtype(a->q_dtype)) return fail(IFA_ERR_PARAM_INVALID, "q_dtype %d not supported", a->q_dtype);
  if (!is_float_dtype(a->out_dtype)) return fail(IFA_ERR_PARAM_INVALID, "out_dtype %d not supported", a->out_dtype);
  if (a->kv_dtype == IFA_I8) {
    if (a->antiquant_scale == nullptr || a->antiquant_offset == nullptr)
      return fail(IFA_ERR_PARAM_NULLPTR, "int8 KV needs antiquant_scale and antiquant_offset");
    if (a->antiquant_mode < IFA_ANTIQUANT_PER_CHANNEL || a->antiquant_mode > IFA_ANTIQUANT_PER_TOKEN_HEAD)
      return fail(IFA_ERR_PARAM_INVALID, "antiquant_mode %d not supported", a->antiquant_mode);
    if (a->antiquant_mode >= IFA_ANTIQUANT_PER_TOKEN && a->qk_dim != 128)
      return fail(IFA_ERR_PARAM_INVALID, "per-token antiquant needs qk_dim 128");
  } else if (a->antiquant_mode != 0) {
    return fail(IFA_ERR_PARAM_INVALID, "antiquant_mode is set for a non-int8 KV cache");
  } else if (!is_float_dtype(a->kv_dtype)) {
    return fail(IFA_ERR_PARAM_INVALID, "kv_dtype %d not supported", a->kv_dtype);
  } else if (a->kv_dtype != a->q_dtype) {
    return fail(IFA_ERR_PARAM_INVALID, "float KV must have the query dtype");
  } else if (a->antiquant_scale || a->antiquant_offset) {
    return fail(IFA_ERR_PARAM_INVALID, "antiquant parameters given for a non-int8 KV cache");
  }
  if (a->kv_layout != IFA_KV_BNSD && a->kv_layout != IFA_KV_PAGED && a->kv_layout != IFA_KV_PAGED_BSH &&
      a->kv_layout != IFA_KV_BSND)
    return fail(IFA_ERR_PARAM_INVALID, "kv_layout %d not supported", a->kv_layout);
  if (a->reserved != 0) return fail(IFA_ERR_PARAM_INVALID, "reserved field must be 0");
  if (a->q_seq_len < 0 || a->q_seq_len > 16)
    return fail(IFA_ERR_PARAM_INVALID, "q_seq_len %lld outside [0, 16]", (long long)a->q_seq_len);
  const int q_seq = a->q_seq_len == 0 ? 1 : (int)a->q_seq_len;
  if (a->sparse_mode != IFA_MASK_NONE && a->sparse_mode != IFA_MASK_CAUSAL && a->sparse_mode != IFA_MASK_TREE)
    return fail(IFA_ERR_PARAM_INVALID, "sparse_mode %d not supported (0, 3 or 9)", a->sparse_mode);
  if (a->num_splits < 0 || a->num_splits > kMaxSplits)
    return fail(IFA_ERR_PARAM_INVALID, "num_splits %d outside [0, %d]", a->num_splits, kMaxSplits);

  // head dims: (64|128, same) through the VALU path, (576, 512) with V
  // aliasing K through the MLA path
  const bool alias = a->value_cache != nullptr && a->value_cache == a->key_cache;
  Path path;
  if (a->qk_dim == 576 && a->v_dim == 512) {
    if (!alias) return fail(IFA_ERR_PARAM_INVALID, "qk_dim 576 / v_dim 512 needs value_cache == key_cache");
    if (a->kv_dtype != IFA_BF16) return fail(IFA_ERR_PARAM_INVALID, "the MLA shape supports bf16 only");
    if (n_kv != 1) return fail(IFA_ERR_PARAM_INVALID, "the MLA shape needs num_key_value_heads 1");
    if (!ifa::mla_supported((int)a->num_heads))
      return fail(IFA_ERR_PARAM_INVALID, "the MLA shape needs num_heads to be a multiple of 32");
    if (q_seq != 1 || a->sparse_mode != IFA_MASK_NONE)
      return fail(IFA_ERR_PARAM_INVALID, "multi-token decode and masks are supported on the GQA shapes only");
    path = Path::kMla;
  } else if ((a->qk_dim == 64 || a->qk_dim == 128) && a->v_dim == a->qk_dim) {
    if (alias) return fail(IFA_ERR_PARAM_INVALID, "value_cache may equal key_cache only for the MLA shape");
    path = Path::kGqa;
  } else {
    return fail(IFA_ERR_PARAM_INVALID, "head dims (qk %lld, v %lld) not supported: use (64,64), (128,128) or (576,512)",
                (long long)a->qk_dim, (long long)a->v_dim);
  }

  int64_t max_len = 0;
  if (is_paged(a->kv_layout)) {
    const int align = a->kv_dtype == IFA_I8 ? 32 : 16;
    if (a->block_size < 16 || a->block_size > 1024 || a->block_size % align)
      return fail(IFA_ERR_PARAM_INVALID, "block_size %lld must be a multiple of %d in [16, 1024]",
                  (long long)a->block_size, align);
    if (a->max_blocks_per_seq < 1) return fail(IFA_ERR_PARAM_INVALID, "max_blocks_per_seq must be >= 1");
    if (a->num_blocks < 1 || a->num_blocks > (int64_t)1 << 31)
      return fail(IFA_ERR_PARAM_INVALID, "num_blocks %lld outside [1, 2^31]", (long long)a->num_blocks);
    max_len = a->max_blocks_per_seq * a->block_size;
    if (max_len > (int64_t)1 << 30) return fail(IFA_ERR_PARAM_INVALID, "max_blocks_per_seq * block_size too large");
    if (a->num_blocks * n_kv * a->block_size >= (int64_t)1 << 32)
      return fail(IFA_ERR_PARAM_INVALID, "the KV pool holds 2^32 or more token rows");
  } else {
    if (a->s_cap < 1 || a->s_cap > (int64_t)1 << 30)
      return fail(IFA_ERR_PARAM_INVALID, "s_cap %lld outside [1, 2^30]", (long long)a->s_cap);
    if (a->batch * n_kv * a->s_cap >= (int64_t)1 << 32)
      return fail(IFA_ERR_PARAM_INVALID, "the KV buffer holds 2^32 or more token rows");
    max_len = a->s_cap;
  }
  if (!std::isfinite(a->scale_value)) return fail(IFA_ERR_PARAM_INVALID, "scale_value is not finite");

  if (a->batch > 0) {
    if (!a->query) return fail(IFA_ERR_PARAM_NULLPTR, "query is NULL");
    if (!a->key_cache) return fail(IFA_ERR_PARAM_NULLPTR, "key_cache is NULL");
    if (!a->value_cache) return fail(IFA_ERR_PARAM_NULLPTR, "value_cache is NULL");
    if (!a->actual_seq_lengths) return fail(IFA_ERR_PARAM_NULLPTR, "actual_seq_lengths is NULL");
    if (!a->attention_out) return fail(IFA_ERR_PARAM_NULLPTR, "attention_out is NULL");
    if (is_paged(a->kv_layout) && !a->block_table)
      return fail(IFA_ERR_PARAM_NULLPTR, "block_table is NULL in the paged layout");
    if (a->sparse_mode == IFA_MASK_TREE && !a->tree_mask)
      return fail(IFA_ERR_PARAM_NULLPTR, "tree_mask is NULL with IFA_MASK_TREE");
  }

  Plan p{};
  p.path = path;
  p.n_kv = n_kv;
  p.group = (int)(a->num_heads / n_kv);
  p.q_seq = q_seq;
  if (path == Path::kGqa) {
    // a workgroup takes gh of the q_seq * group query rows of a KV head
    const int rows_kv = q_seq * p.group;
    const int gh_max = ifa::gqa_max_heads_per_wg(a->kv_dtype, (int)a->qk_dim);
    int gh = 1;
    for (int c = gh_max; c >= 1; c >>= 1)
      if (rows_kv % c == 0) { gh = c; break; }
    p.heads_per_wg = gh;
    if (!ifa::gqa_supported(a->q_dtype, a->kv_dtype, (int)a->qk_dim, gh))
      return fail(IFA_ERR_PARAM_INVALID, "dtype combination (q %d, kv %d) not supported", a->q_dtype, a->kv_dtype);
    // 16-bit K/V with head dim 128: the rows of a KV head (any number of
    // query tokens) go to the matrix cores in groups of 32, one wave each
    p.mfma = ifa::gqa_mfma_supported(a->q_dtype, a->kv_dtype, (int)a->qk_dim);
    if (p.mfma) {
      p.heads_per_wg = 32;
      p.balanced = use_balanced_gqa(a, rows_kv, max_len);
      p.n_split = p.balanced ? balanced_runs_gqa(a, n_kv, rows_kv, max_len)
                             : (a->num_splits ? a->num_splits : auto_splits_mfma(a, n_kv, rows_kv, max_len));
    } else {
      p.n_split = a->num_splits ? a->num_splits : auto_splits_gqa(a, n_kv, rows_kv, gh, max_len);
    }
  } else {
    p.heads_per_wg = (int)a->num_heads;
    p.balanced = use_balanced_mla(a, max_len);
    p.n_split = p.balanced ? balanced_runs(a) : (a->num_splits ? a->num_splits : auto_splits_mla(a, max_len));
    if (!p.balanced && (p.n_split > kMaxSplits || p.n_split < min_splits_mla(a, max_len)))
      return fail(IFA_ERR_PARAM_INVALID,
                  "the MLA shape needs num_splits >= %lld so that a split spans at most %d cache blocks",
                  (long long)min_splits_mla(a, max_len), ifa::kMlaMaxTableSlice - 2);
  }
  // partial rows: (sequence, query token, head, split), or (slot, query
  // token, head) with runs + batch slots in the balanced split
  const size_t rows = p.balanced ? ((size_t)p.n_split + (size_t)a->batch) * (size_t)q_seq * (size_t)a->num_heads
                                 : (size_t)a->batch * (size_t)q_seq * (size_t)a->num_heads * (size_t)p.n_split;
  p.off_o = 0;
  // partial outputs: fp32, fp16 on the MLA path
  p.off_m = align256(rows * (size_t)a->v_dim * (p.path == Path::kMla ? 2 : sizeof(float)));
  p.off_l = p.off_m + align256(rows * sizeof(float));
  p.off_plan = p.off_l + align256(rows * sizeof(float));
  // longest-first plan: (sequence, clamped length) per rank, int32 pairs; in
  // the balanced split, (first slot, slot count) per sequence
  p.bytes = p.off_plan + (a->batch <= ifa::kLongestFirstMaxBatch ? align256((size_t)a->batch * 8) : 0);
  if (rows == 0) p.bytes = 0;
  *plan = p;
  return IFA_OK;
}

ifa_status check_workspace(const Plan& p, const void* ws, size_t ws_bytes) {
  if (ws_bytes < p.bytes)
    return fail(IFA_ERR_PLAN, "workspace of %zu bytes is smaller than the %zu bytes needed", ws_bytes, p.bytes);
  if (p.bytes && !ws) return fail(IFA_ERR_PARAM_NULLPTR, "workspace is NULL");
  if (p.bytes && (reinterpret_cast<uintptr_t>(ws) & 255))
    return fail(IFA_ERR_PARAM_INVALID, "workspace must be 256-byte aligned");
  return IFA_OK;
}

ifa_status runtime(hipError_t e, const char* what) {
  if (e == hipSuccess) return IFA_OK;
  return fail(IFA_ERR_RUNTIME, "%s: %s", what, hipGetErrorString(e));
}

ifa_status run_splitkv(const ifa_decode_args* a, const Plan& p, void* ws, hipStream_t stream,
                       const ifa::LaunchEvents* ev = nullptr) {
  char* w = static_cast<char*>(ws);
  const int64_t max_len = is_paged(a->kv_layout) ? a->max_blocks_per_seq * a->block_size : a->s_cap;
  // Longest-first order for batches of up to 256 sequences.  The int8-KV GQA
  // kernel, with twice the workgroups and each one's start not hidden behind
  // streaming, takes it from a planning kernel launched first; the 16-bit GQA
  // and MLA workgroups rank the lengths themselves, which costs less than the
  // extra launch there.
  const bool longest_first = a->batch <= ifa::kLongestFirstMaxBatch;
  const bool use_plan = longest_first && p.path == Path::kGqa && a->kv_dtype == IFA_I8 && !p.mfma;
  int2* plan = nullptr;
  if (use_plan) {
    plan = reinterpret_cast<int2*>(w + p.off_plan);
    ifa_status st = runtime(ifa::launch_plan(a->actual_seq_lengths, (int)a->batch, max_len, plan, stream),
                            "planning launch");
    if (st != IFA_OK) return st;
  }
  const float scale_log2 = (float)(a->scale_value * 1.4426950408889634);
  if (p.path == Path::kGqa) {
    ifa::GqaLaunch L{};
    L.q = a->query;
    L.k = a->key_cache;
    L.v = a->value_cache;
    L.block_table = a->block_table;
    L.seq_lens = a->actual_seq_lengths;
    L.aq_scale = a->antiquant_scale;
    L.aq_offset = a->antiquant_offset;
    L.ws_o = reinterpret_cast<float*>(w + p.off_o);
    L.ws_m = reinterpret_cast<float*>(w + p.off_m);
    L.ws_l = reinterpret_cast<float*>(w + p.off_l);
    L.batch = (int)a->batch;
    L.n_q = (int)a->num_heads;
    L.n_kv = (int)p.n_kv;
    L.group = p.group;
    L.heads_per_wg = p.heads_per_wg;
    L.q_seq = p.q_seq;
    L.rows_kv = p.q_seq * p.group;
    L.mask_mode = a->sparse_mode;
    L.tree_mask = a->tree_mask;
    L.n_split = p.n_split;
    L.s_cap = max_len;
    L.block_size = (int)a->block_size;
    L.max_blocks = (int)a->max_blocks_per_seq;
    L.num_blocks = (int)a->num_blocks;
    L.paged = is_paged(a->kv_layout);
    L.token_major = is_token_major(a->kv_layout);
    // antiquant parameter strides (entries; K/V index, KV head, channel)
    const bool per_tensor = a->antiquant_mode == IFA_ANTIQUANT_PER_TENSOR;
    L.aq_stride_kv = per_tensor ? 1 : (int)(p.n_kv * a->qk_dim);
    L.aq_stride_g = per_tensor ? 0 : (int)a->qk_dim;
    L.aq_stride_d = per_tensor ? 0 : 1;
    // per token: (2, B, S) or (2, B, N_kv, S) over the logical positions S = max_len
    L.aq_token = a->kv_dtype == IFA_I8 && a->antiquant_mode >= IFA_ANTIQUANT_PER_TOKEN;
    if (L.aq_token) {
      const int64_t heads = a->antiquant_mode == IFA_ANTIQUANT_PER_TOKEN_HEAD ? p.n_kv : 1;
      L.aq_tok_stride_g = heads > 1 ? max_len : 0;
      L.aq_tok_stride_b = heads * max_len;
      L.aq_tok_stride_kv = a->batch * heads * max_len;
    }
    L.scale_log2 = scale_log2;
    if (L.paged) ifa::make_divisor((uint32_t)a->block_size, &L.bs_magic, &L.bs_shift);
    L.plan = plan;
    L.longest_first = longest_first;
    L.balanced = p.balanced;
    L.seg_desc = p.balanced ? reinterpret_cast<int2*>(w + p.off_plan) : nullptr;
    L.q_dtype = a->q_dtype;
    L.kv_dtype = a->kv_dtype;
    L.head_dim = (int)a->qk_dim;
    if (p.mfma) return runtime(ifa::launch_gqa_mfma(L, stream, ev), "multi-token split-KV decode launch");
    return runtime(ifa::launch_gqa_splitkv(L, stream, ev), "split-KV decode launch");
  }
  ifa::MlaLaunch M{};
  M.q = a->query;
  M.kv = a->key_cache;
  M.block_table = a->block_table;
  M.seq_lens = a->actual_seq_lengths;
  M.ws_o = reinterpret_cast<_Float16*>(w + p.off_o);
  M.ws_m = reinterpret_cast<float*>(w + p.off_m);
  M.ws_l = reinterpret_cast<float*>(w + p.off_l);
  M.batch = (int)a->batch;
  M.n_q = (int)a->num_heads;
  M.n_split = p.n_split;
  M.s_cap = max_len;
  M.block_size = (int)a->block_size;
  M.max_blocks = (int)a->max_blocks_per_seq;
  M.num_blocks = (int)a->num_blocks;
  M.scale_log2 = scale_log2;
  // one KV head: the token-major layouts address exactly as the head-major ones
  if (is_paged(a->kv_layout)) ifa::make_divisor((uint32_t)a->block_size, &M.bs_magic, &M.bs_shift);
  M.longest_first = longest_first;
  M.qk_dim = (int)a->qk_dim;
  M.v_dim = (int)a->v_dim;
  M.paged = is_paged(a->kv_layout);
  M.balanced = p.balanced;
  M.seg_desc = p.balanced ? reinterpret_cast<int2*>(w + p.off_plan) : nullptr;
  return runtime(ifa::launch_mla_splitkv(M, stream, ev), "MLA split-KV decode launch");
}

ifa_status run_combine(const ifa_decode_args* a, const Plan& p, const void* ws, hipStream_t stream) {
  const char* w = static_cast<const char*>(ws);
  ifa::CombineLaunch C{};
  C.ws_o = w + p.off_o;
  C.o_f16 = p.path == Path::kMla;
  C.ws_m = reinterpret_cast<const float*>(w + p.off_m);
  C.ws_l = reinterpret_cast<const float*>(w + p.off_l);
  C.seq_lens = a->actual_seq_lengths;
  C.sink = a->learnable_sink;
  C.out = a->attention_out;
  C.lse = a->softmax_lse;
  C.batch = (int)a->batch * p.q_seq;  // rows are (sequence, query token, head)
  C.q_seq = p.q_seq;
  C.n_q = (int)a->num_heads;
  C.n_split = p.n_split;
  C.v_dim = (int)a->v_dim;
  C.out_dtype = a->out_dtype;
  C.s_cap = is_paged(a->kv_layout) ? a->max_blocks_per_seq * a->block_size : a->s_cap;
  C.seg_desc = p.balanced ? reinterpret_cast<const int2*>(w + p.off_plan) : nullptr;
  return runtime(ifa::launch_combine(C, stream), "combine launch");
}

}  // namespace

namespace ifa {
ifa_status set_last_error(ifa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}
}  // namespace ifa

extern "C" {

ifa_status ifa_decode_workspace_size(const ifa_decode_args* args, size_t* workspace_bytes) {
  if (!workspace_bytes) return fail(IFA_ERR_PARAM_NULLPTR, "workspace_bytes is NULL");
  Plan p;
  ifa_status st = validate_and_plan(args, &p);
  if (st != IFA_OK) return st;
  *workspace_bytes = p.bytes;
  return ok();
}

ifa_status ifa_decode_num_splits(const ifa_decode_args* args, int32_t* num_splits) {
  if (!num_splits) return fail(IFA_ERR_PARAM_NULLPTR, "num_splits is NULL");
  Plan p;
  ifa_status st = validate_and_plan(args, &p);
  if (st != IFA_OK) return st;
  *num_splits = p.n_split;
  return ok();
}

ifa_status ifa_decode_split_mode(const ifa_decode_args* args, int32_t* balanced) {
  if (!balanced) return fail(IFA_ERR_PARAM_NULLPTR, "balanced is NULL");
  Plan p;
  ifa_status st = validate_and_plan(args, &p);
  if (st != IFA_OK) return st;
  *balanced = p.balanced ? 1 : 0;
  return ok();
}

ifa_status ifa_decode_splitkv(const ifa_decode_args* args, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  Plan p;
  ifa_status st = validate_and_plan(args, &p);
  if (st != IFA_OK) return st;
  if ((st = check_workspace(p, workspace, workspace_bytes)) != IFA_OK) return st;
  if (args->batch == 0) return ok();
  if ((st = run_splitkv(args, p, workspace, stream)) != IFA_OK) return st;
  return ok();
}

ifa_status ifa_decode_splitkv_timed(const ifa_decode_args* args, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  if (!start || !stop) return fail(IFA_ERR_PARAM_NULLPTR, "start and stop events are required");
  Plan p;
  ifa_status st = validate_and_plan(args, &p);
  if (st != IFA_OK) return st;
  if ((st = check_workspace(p, workspace, workspace_bytes)) != IFA_OK) return st;
  if (args->batch == 0) return ok();
  const ifa::LaunchEvents ev{start, stop};
  if ((st = run_splitkv(args, p, workspace, stream, &ev)) != IFA_OK) return st;
  return ok();
}

ifa_status ifa_decode_combine(const ifa_decode_args* args, const void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  Plan p;
  ifa_status st = validate_and_plan(args, &p);
  if (st != IFA_OK) return st;
  if ((st = check_workspace(p, workspace, workspace_bytes)) != IFA_OK) return st;
  if (args->batch == 0) return ok();
  if ((st = run_combine(args, p, workspace, stream)) != IFA_OK) return st;
  return ok();
}

ifa_status ifa_decode(const ifa_decode_args* args, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Plan p;
  ifa_status st = validate_and_plan(args, &p);
  if (st != IFA_OK) return st;
  if ((st = check_workspace(p, workspace, workspace_bytes)) != IFA_OK) return st;
  if (args->batch == 0) return ok();
  if ((st = run_splitkv(args, p, workspace, stream)) != IFA_OK) return st;
  if ((st = run_combine(args, p, workspace, stream)) != IFA_OK) return st;
  return ok();
}

ifa_status attn_update(const void* prev_attn_out, const float* prev_softmax_max, const float* prev_softmax_sum,
                       const void* cur_attn_out, const float* cur_softmax_max, const float* cur_softmax_sum,
                       void* attn_out, float* softmax_max_out, float* softmax_sum_out, int64_t rows,
                       int64_t head_dim, int32_t dtype, int32_t stat_stride, hipStream_t stream) {
  if (rows < 0) return fail(IFA_ERR_PARAM_INVALID, "rows must be >= 0");
  if (head_dim < 1 || head_dim > 65536) return fail(IFA_ERR_PARAM_INVALID, "head_dim outside [1, 65536]");
  if (!is_float_dtype(dtype)) return fail(IFA_ERR_PARAM_INVALID, "dtype %d not supported", dtype);
  if (stat_stride != 1 && stat_stride != 8) return fail(IFA_ERR_PARAM_INVALID, "stat_stride must be 1 or 8");
  if (rows == 0) return ok();
  if (!prev_attn_out || !prev_softmax_max || !prev_softmax_sum || !cur_attn_out || !cur_softmax_max ||
      !cur_softmax_sum || !attn_out || !softmax_max_out || !softmax_sum_out)
    return fail(IFA_ERR_PARAM_NULLPTR, "attn_update: a required pointer is NULL");
  ifa::UpdateLaunch U{};
  U.prev_out = prev_attn_out;
  U.prev_max = prev_softmax_max;
  U.prev_sum = prev_softmax_sum;
  U.cur_out = cur_attn_out;
  U.cur_max = cur_softmax_max;
  U.cur_sum = cur_softmax_sum;
  U.out = attn_out;
  U.max_out = softmax_max_out;
  U.sum_out = softmax_sum_out;
  U.rows = rows;
  U.head_dim = (int)head_dim;
  U.dtype = dtype;
  U.stat_stride = stat_stride;
  ifa_status st = runtime(ifa::launch_update(U, stream), "attn_update launch");
  if (st != IFA_OK) return st;
  return ok();
}

ifa_status ifa_kv_cache_write(const void* src, const int64_t* slot_index, void* cache, int64_t tokens,
                              int64_t num_kv_heads, int64_t d, int64_t row_elems, int64_t col_offset,
                              int64_t num_blocks, int64_t block_size, int32_t layout, int32_t dtype,
                              hipStream_t stream) {
  if (tokens < 0) return fail(IFA_ERR_PARAM_INVALID, "tokens must be >= 0");
  if (num_kv_heads < 1 || num_kv_heads > 256) return fail(IFA_ERR_PARAM_INVALID, "num_kv_heads outside [1, 256]");
  if (d < 1 || col_offset < 0 || row_elems < col_offset + d || row_elems > 65536)
    return fail(IFA_ERR_PARAM_INVALID, "need 1 <= d, 0 <= col_offset, col_offset + d <= row_elems <= 65536");
  if (num_blocks < 1 || block_size < 1 || block_size > 1024)
    return fail(IFA_ERR_PARAM_INVALID, "num_blocks must be >= 1 and block_size in [1, 1024]");
  if (layout != IFA_KV_PAGED && layout != IFA_KV_PAGED_BSH)
    return fail(IFA_ERR_PARAM_INVALID, "layout %d is not a paged layout", layout);
  if (dtype != IFA_F32 && dtype != IFA_F16 && dtype != IFA_BF16 && dtype != IFA_I8)
    return fail(IFA_ERR_PARAM_INVALID, "dtype %d not supported", dtype);
  const int64_t esz = dtype == IFA_F32 ? 4 : (dtype == IFA_I8 ? 1 : 2);
  if ((d * esz) % 16 || (col_offset * esz) % 16 || (row_elems * esz) % 16)
    return fail(IFA_ERR_PARAM_INVALID, "d, col_offset and row_elems must each span a multiple of 16 bytes");
  if (tokens == 0) return ok();
  if (!src || !slot_index || !cache) return fail(IFA_ERR_PARAM_NULLPTR, "ifa_kv_cache_write: a pointer is NULL");
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(cache)) & 15)
    return fail(IFA_ERR_PARAM_INVALID, "src and cache must be 16-byte aligned");
  ifa::CacheWriteLaunch W{};
  W.src = src;
  W.slot_index = slot_index;
  W.cache = cache;
  W.tokens = tokens;
  W.n_kv = num_kv_heads;
  W.row_chunks = d * esz / 16;
  W.row_bytes = row_elems * esz;
  W.col_bytes = col_offset * esz;
  W.num_blocks = num_blocks;
  W.block_size = block_size;
  W.token_major = layout == IFA_KV_PAGED_BSH;
  ifa_status st = runtime(ifa::launch_cache_write(W, stream), "cache write launch");
  if (st != IFA_OK) return st;
  return ok();
}

int64_t ifa_paged_block_count(const int64_t* lengths, int64_t batch, int64_t block_size) {
  if (!lengths || batch < 0 || block_size < 1) return -1;
  int64_t total = 0;
  for (int64_t b = 0; b < batch; ++b) {
    if (lengths[b] < 0) return -1;
    total += (lengths[b] + block_size - 1) / block_size;
  }
  return total;
}

ifa_status ifa_decode_check_inputs(const ifa_decode_args* args, int32_t* flags, hipStream_t stream) {
  if (!flags) return fail(IFA_ERR_PARAM_NULLPTR, "flags is NULL");
  Plan p;
  ifa_status st = validate_and_plan(args, &p);
  if (st != IFA_OK) return st;
  ifa::CheckLaunch C{};
  C.seq_lens = args->actual_seq_lengths;
  C.block_table = is_paged(args->kv_layout) ? args->block_table : nullptr;
  C.flags = flags;
  C.batch = args->batch;
  C.block_size = is_paged(args->kv_layout) ? args->block_size : 1;
  C.max_blocks = is_paged(args->kv_layout) ? args->max_blocks_per_seq : 0;
  C.s_cap = is_paged(args->kv_layout) ? args->max_blocks_per_seq * args->block_size : args->s_cap;
  C.num_blocks = args->num_blocks;
  if ((st = runtime(ifa::launch_check(C, stream), "input check launch")) != IFA_OK) return st;
  return ok();
}

ifa_status ifa_read_bandwidth_probe(const void* buf, size_t bytes, uint32_t* out, int32_t workgroups,
                                    hipStream_t stream) {
  if (workgroups < 1 || workgroups > (1 << 20)) return fail(IFA_ERR_PARAM_INVALID, "workgroups outside [1, 2^20]");
  if (bytes % 16) return fail(IFA_ERR_PARAM_INVALID, "bytes must be a multiple of 16");
  if (bytes == 0) return ok();
  if (!buf || !out) return fail(IFA_ERR_PARAM_NULLPTR, "ifa_read_bandwidth_probe: a pointer is NULL");
  if (reinterpret_cast<uintptr_t>(buf) & 15) return fail(IFA_ERR_PARAM_INVALID, "buf must be 16-byte aligned");
  ifa_status st = runtime(ifa::launch_read_probe(buf, bytes, out, workgroups, stream), "read probe launch");
  if (st != IFA_OK) return st;
  return ok();
}

const char* ifa_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
