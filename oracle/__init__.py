"""CPU oracle for the DSA hot path (index scores, top-k selection, sparse
MQA attention), in float64 from the definitions on the pages.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in
this package.  It shares no code, header, table or helper with the HIP
library (``long_context_02_amd``) and imports nothing from it.

Parity status of each function (pins live in ``tests/test_oracle_*.py``):
  fp8.e4m3_decode / e4m3_encode   pinned (torch's e4m3fn cast, exhaustive)
  fp8.quantize_rows               pinned (amax element -> +-448, power-of-two
                                  scale invariance, zero rows, half-step error)
  cache_append                    pinned (untouched rows, per-sequence
                                  positions, skipped out-of-range rows)
  indexer_kl (dense, sparse)      pinned (torch kl_div + float64 autograd,
                                  p = softmax(I) gives 0, one-hot closed form,
                                  finite differences, shift invariance,
                                  sparse over all candidates equals dense)
  index_scores                    pinned (hand 4-token example, integer dot
                                  identity, pure-Python brute force)
  topk_select                     pinned (full sort by (score desc, index asc),
                                  hand example, constructed ties)
  sparse_mqa_attention            pinned (k >= L equals dense causal attention
                                  from torch SDPA; q = 0 mean; single index;
                                  permutation and duplicate closed forms)
  sparse_mqa_attention_bwd        pinned (central finite differences of the
                                  forward, float64 autograd through torch
                                  SDPA when k >= L, gradient sums
                                  sum_h dq.q = sum_i dc_i.c_i, duplicates)
  sparse_mha_attention            pinned (absorption identity against the
                                  MQA-mode oracle; k >= L equals dense causal
  mha_keys_values                 multi-head attention from torch SDPA with
                                  per-head keys and values; single index
                                  gives that head's value row)
  dsa_forward                     pinned (composition; chunked prefill equals
                                  the tail rows of a full prefill)
"""
from .fp8 import e4m3_decode, e4m3_encode, dequantize, quantize_rows, E4M3_MAX  # noqa: F401
from .dsa import (  # noqa: F401
    index_scores,
    index_scores_row,
    topk_select,
    topk_select_row,
    sparse_mqa_attention,
    sparse_mqa_attention_row,
    sparse_mqa_attention_bwd,
    sparse_mqa_attention_bwd_row,
    mha_keys_values,
    sparse_mha_attention,
    sparse_mha_attention_row,
    dsa_forward,
    cache_append,
    indexer_kl,
    indexer_kl_dense_row,
    indexer_kl_sparse_row,
)
