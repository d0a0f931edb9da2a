"""Parameter counting for MoE transformer shapes (TEST INFRASTRUCTURE).

Pins the Mixtral-shaped workload against the exact counts printed in the
"Week 2 Day 2: Mixture of Experts" course notes (semidirectx.com, CME295),
§2.1, and the CMU 15-779 Lecture 21 notes, §10 exercise 1.
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class ModelShape:
    layers: int
    d: int
    q_heads: int
    kv_heads: int
    head_dim: int
    E: int
    k: int
    d_ff: int
    vocab: int
    n_shared: int = 0
    tied_embeddings: bool = False
    norms_per_layer: int = 2        # RMSNorm weight vectors per block
    final_norm: bool = True


def attention_params(m: ModelShape) -> int:
    """Q and O are d x (q_heads*head_dim); K and V are d x (kv_heads*head_dim); no bias."""
    return 2 * m.d * m.q_heads * m.head_dim + 2 * m.d * m.kv_heads * m.head_dim


def expert_params(m: ModelShape) -> int:
    """A SwiGLU expert has three d x d_ff matrices and no bias."""
    return 3 * m.d * m.d_ff


def router_params(m: ModelShape) -> int:
    return m.d * m.E


def counts(m: ModelShape, with_norms: bool = True):
    """(total, active-per-token) parameter counts."""
    emb = m.vocab * m.d * (1 if m.tied_embeddings else 2)
    norms = (m.layers * m.norms_per_layer * m.d + (m.d if m.final_norm else 0)) if with_norms else 0
    per_layer_total = attention_params(m) + (m.E + m.n_shared) * expert_params(m) + router_params(m)
    per_layer_active = attention_params(m) + (m.k + m.n_shared) * expert_params(m) + router_params(m)
    return (m.layers * per_layer_total + emb + norms,
            m.layers * per_layer_active + emb + norms)


MIXTRAL_8X7B = ModelShape(layers=32, d=4096, q_heads=32, kv_heads=8, head_dim=128,
                          E=8, k=2, d_ff=14336, vocab=32000)
