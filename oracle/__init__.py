"""Float64 CPU oracle for paged split-KV decode attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this package.  The GPU library never
calls it, and it shares no code, tables or helpers with the GPU path.

Every function is the plain definition from the pages, in NumPy float64:

* attention: aclnnIncreFlashAttentionV3, "Function" section, self-attention
  formula Softmax(Q K^T / sqrt(d)) V, with S of the query fixed to 1;
* learnable sink: aclnnFlashAttentionScoreV4, "计算公式" (formula) section,
  m = max(sink, max S), out = sum e^(S-m) V / (sum e^(S-m) + e^(sink-m));
* merge of two partial results: aclnnRingAttentionUpdate, "功能说明" formula,
  read in its sum-weighted form (see ``merge``);
* paged gather: aclnnIncreFlashAttentionV3, "Constraints", page attention
  scenario (blockTable, blockSize, KV layout (blocknum, KV_N, blocksize, D));
* block count: aclnnMlaPrologV3WeightNz, "Constraints", BlockNum row;
* paged KV-cache write: aclnnMlaPrologV3WeightNz, "Parameters", kvCacheRef /
  cacheIndexOptional (``cache_ref.cache_write``);
* multi-token decode with the rightDownCausal and treeMask masks of the
  FusedInferAttentionScore blog (``spec_ref.decode_multi``).

Parity pins: every function here is pinned by the CPU tests in
tests/test_oracle_pins.py.  Three readings are not fixed by the pages and are
therefore "parity unpinned" as to convention (the oracle and the GPU path share
the reading): the antiquant offset sign, the GQA head-to-group mapping, and the
sign of the log-sum-exp for an empty sequence.
"""

from .attn_ref import (  # noqa: F401
    as_f64,
    gather_kv,
    dequant,
    softmax_weights,
    attention_row,
    partial_triple,
    merge,
    merge_many,
    decode,
    decode_rows,
    decode_workload,
    attn_update,
    block_count,
    lengths_from_prefix_sums,
)
from .cache_ref import cache_write  # noqa: F401,E402
from .spec_ref import MASK_CAUSAL, MASK_NONE, MASK_TREE, decode_multi, visible_tokens  # noqa: F401,E402
