"""Plain CPU oracle for the Memory Sparse Attention (MSA) hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library: it has its own bf16 widening, its own RoPE, its own pooling, routing,
top-k and attention, all written as the plain definitions in float64 NumPy.

Sources (the pages the method is taken from):

* neo-ai.one article on MSA, section 全体設計 › アーキテクチャ (Fig. 2): chunk
  mean-pooling of K/V/Kr, cosine routing (mean over heads, then max over
  tokens), top-k documents, concatenation with the local K/V; document-wise
  RoPE restarting at 0; global RoPE shifting the query start by k.
* same article, section 推論パイプライン (Fig. 3): offline encode -> online
  routing and context assembly -> sparse generation; K̄r on the GPU, K̄/V̄ in
  host memory fetched on demand.
* ruixiangma.github.io blog "Memory-Sparse-Attention", 方法 › 稀疏注意力机制
  (fixed-length chunks, mean pooling, cosine top-k documents) and 文档级RoPE.
* github-eval-reports review of MSA, 核心模块 (head mean first, then token max)
  and 核心能力 › 端到端可训练框架 (one differentiable loop); the blog's 训练策略
  (generation loss plus an auxiliary routing loss) for the backward.

Every reading taken where the pages are silent is listed in the module that
takes it.  Parity status of each function is stated in its module docstring.
"""

from .bf16 import bf16_bits_to_f64, f64_to_bf16_bits, f32_to_f64
from .rope import inv_freq, rope_angles, rope
from .encode import chunk_counts, chunk_offsets, chunk_mean, encode_pool, encode_pool_loops
from .route import (chunk_scores, chunk_scores_loops, doc_scores,
                    topk_docs, route, EPS)
from .gather import gather_rows
from .attention import sparse_attn, sparse_attn_loops
from .backward import (sparse_attn_lse, sparse_attn_bwd, sparse_attn_bwd_sampled, pair_scores,
                       doc_score_argmax, route_score_bwd, encode_pool_bwd)

__all__ = [
    "bf16_bits_to_f64", "f64_to_bf16_bits", "f32_to_f64",
    "inv_freq", "rope_angles", "rope",
    "chunk_counts", "chunk_offsets", "chunk_mean", "encode_pool", "encode_pool_loops",
    "chunk_scores", "chunk_scores_loops", "doc_scores", "topk_docs",
    "route", "EPS",
    "gather_rows",
    "sparse_attn", "sparse_attn_loops",
    "sparse_attn_lse", "sparse_attn_bwd", "sparse_attn_bwd_sampled", "pair_scores", "doc_score_argmax",
    "route_score_bwd",
    "encode_pool_bwd",
]
