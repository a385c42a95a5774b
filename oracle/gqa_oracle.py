"""fp64 CPU oracle for single-token grouped-query (GQA) decode attention, the comparator.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, calls or links
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` use it. It shares no code with the HIP path.

Where it comes from (page "Multi-Head Low-Rank Attention", ai.info AI summary
of arXiv 2603.02188): GQA is the baseline MLRA-4's decode kernel is compared
against ("Key Contributions" #4), analysed at the shape of a public GQA model
with 64 query heads, 8 KV heads and head dimension 128 ("Methodology in Plain
English", 4th paragraph). The pages do not spell GQA out; this oracle takes the
standard reading: the query heads are cut into H_kv consecutive groups of
G = H_q / H_kv heads, every head of group g attends over KV head g with its own
softmax, and keys and values are separate cached tensors of the same width.

Definition, per sequence b with L = seqlens[b] cached tokens, query head i:

    g        = i // (H_q / H_kv)
    rho(t)   = block_table[b, t // P] * P + t % P   (paged)  |  b * max_seqlen + t
    s_t      = sm_scale * <q[b, i], K[rho(t), g]>
    out[b,i] = sum_t softmax_t(s)_t * V[rho(t), g]

L = 0 gives out[b] = 0. Inputs are promoted exactly to float64; library matrix
products serve as the dot products. The softmax subtracts the exact maximum.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .mlra_oracle import as_f64, physical_rows

__all__ = ["gqa_group_of", "gqa_head_attention", "gqa_decode", "gqa_decode_inputs"]


def gqa_group_of(i: int, num_q_heads: int, num_kv_heads: int) -> int:
    """KV head that query head i reads: heads are grouped in consecutive runs of H_q / H_kv."""
    return i // (num_q_heads // num_kv_heads)


def gqa_head_attention(q_i: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float) -> np.ndarray:
    """softmax_t(sm_scale * <q_i, K_t>) weighted sum of V_t, with the exact max subtracted."""
    s = sm_scale * (K @ q_i)
    w = np.exp(s - s.max())
    return (w @ V) / w.sum()


def gqa_decode(q, k_cache, v_cache, seqlens: Sequence[int], *, sm_scale: float,
               block_table=None, page_size: int = 0, max_seqlen: Optional[int] = None,
               batch_indices: Optional[Sequence[int]] = None) -> np.ndarray:
    """q [B, H_q, D]; k_cache, v_cache [rows, H_kv, D]; returns out [B, H_q, D] float64
    (rows of sequences outside batch_indices stay 0)."""
    seqlens = [int(x) for x in seqlens]
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    if max_seqlen is None:
        max_seqlen = max(seqlens) if seqlens else 0
    bt = None if block_table is None else np.asarray(
        block_table.cpu() if hasattr(block_table, "cpu") else block_table, dtype=np.int64)
    out = np.zeros((B, Hq, v_cache.shape[2]))
    for b in (range(B) if batch_indices is None else batch_indices):
        L = seqlens[b]
        if L == 0:
            continue
        rows = physical_rows(b, L, bt, page_size, max_seqlen)
        K = as_f64(k_cache[rows])
        V = as_f64(v_cache[rows])
        qb = as_f64(q[b])
        for i in range(Hq):
            g = gqa_group_of(i, Hq, Hkv)
            out[b, i] = gqa_head_attention(qb[i], K[:, g, :], V[:, g, :], sm_scale)
    return out


def gqa_decode_inputs(inp, batch_indices=None, **overrides) -> np.ndarray:
    """The oracle on a generated GQA input bundle (mlra_workloads.GqaInputs)."""
    kw = dict(sm_scale=inp.w.sm_scale, block_table=inp.block_table, page_size=inp.w.page_size,
              max_seqlen=inp.max_seqlen, batch_indices=batch_indices)
    kw.update(overrides)
    return gqa_decode(inp.q, inp.k_cache, inp.v_cache, inp.seqlens.tolist(), **kw)
