"""Float64 CPU oracle for jagged generalized dot-product attention (forward).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The GPU library never calls it and
shares no code with it (the seeded input generator is the only common module).

Sources: the three web pages on Meta's GEM ads model --
  [GEM-T]  techfeed.io summary of "GEM Training: How Meta Doubled the Efficiency
           of Its LLM-Scale Ads Foundation Model"
  [GEM-S]  aigeeknews.com "Meta の生成型広告モデル（GEM）：フロンティア広告 AI に向けた
           中央モデルと計算エンジンのスケーリング"
  [GEM-R]  remio.ai "Meta Engineering、広告モデルの拡大とともにGEMの学習効率を2倍にしたと説明"

Every function is pinned by tests/test_oracle_*.py against facts fixed outside
this code (library routines, closed forms, invariants, brute force).  Parity of
the pages' unspecified "6th-order Taylor" GELU approximation is unpinned: the
oracle computes exact gelu_tanh only.
"""
from .gdpa import (gdpa_forward, gdpa_rows, gelu_tanh, rms_normalise,
                   block_window_allowed, sliding_window_allowed, attention_dense, attended_pairs,
                   attention_lse, gdpa_lse)
from .gdpa_bwd import (gdpa_backward, attention_dense_bwd, attention_dense_gelu_bwd, gelu_tanh_grad,
                       rms_normalise_bwd)
from .mx import decode_e4m3, decode_e8m0, mx_dequantise, encode_e4m3, mx_encode, e4m3_grid

__all__ = ["gdpa_backward", "attention_dense_bwd", "attention_dense_gelu_bwd", "gelu_tanh_grad",
           "rms_normalise_bwd", "gdpa_forward", "gdpa_rows", "gelu_tanh", "rms_normalise",
           "block_window_allowed", "sliding_window_allowed", "attention_dense", "attended_pairs",
           "attention_lse", "gdpa_lse",
           "decode_e4m3", "decode_e8m0", "mx_dequantise", "encode_e4m3", "mx_encode", "e4m3_grid"]
