"""fp64 CPU oracle for single-token MLRA / absorbed-MLA decode attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, calls or links
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` use it. It shares no code with the HIP path.

What it computes, and where the pages state it (all citations are to the page
"Multi-Head Low-Rank Attention", ai.info AI summary of arXiv 2603.02188):

* Decoding is three absorbable steps: query-side absorption, MQA-style
  attention over the shared latent cache, and an output up-projection; no
  per-head NoPE key or value is materialised ("Main Findings", 4th bullet).
  The query handed to this oracle is already absorbed: q_nope[b, i, j] lives
  in latent coordinates of latent head j.
* MLRA splits the latent into NB latent heads, runs attention on each one
  separately and sums the NB attention outputs, each up-projected by its own
  value block ("Key Contributions" #2; "Methodology in Plain English",
  2nd paragraph). The branches have separate softmaxes.
* The per-branch logit space after absorption is 1.5 d_h = 128 latent + 64
  RoPE channels ("Key Contributions" #2): every branch adds the same RoPE
  logit <q_rope, k_rope> of its query head.
* The summed outputs are rescaled for the branch count: 1/2 for four branches,
  1/sqrt(2) for two ("Key Contributions" #3); MLA (one latent, no branch sum)
  uses 1.

Definition, per sequence b with L = seqlens[b] cached tokens (the new token
already appended), for every query head i:

    rho(t)   = block_table[b, t // P] * P + t % P   (paged)  |  b * max_seqlen + t
    u_t      = <q_rope[b,i], R[rho(t)]>                      shared by all branches
    s_{j,t}  = sm_scale * (<q_nope[b,i,j], C[rho(t), j]> + u_t)
    obar_j   = sum_t softmax_t(s_j)_t * C[rho(t), j]         in R^{D_L}
    out[b,i] = out_scale * sum_j obar_j @ W_UV[j, i]          W_UV[j,i] in R^{D_L x D_V}

L = 0 gives out[b] = 0. All inputs are promoted exactly to float64; library
matrix products serve as the dot products. ``decode_split`` is the split-KV
reformulation (per-chunk running max / sum / unnormalised output, merged with
log-sum-exp weights), which is exact and is pinned against ``decode``.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

try:  # torch is only needed to read bf16 storage
    import torch
except Exception:  # pragma: no cover
    torch = None

__all__ = [
    "as_f64", "physical_rows", "rope_scores", "branch_scores", "softmax_average",
    "up_project", "branch_sum", "decode", "decode_split", "decode_inputs", "partial_stats", "merge_partials",
    "absorb",
]


def as_f64(x) -> np.ndarray:
    """Exact promotion of bf16 / fp32 / fp64 storage (torch or numpy) to float64."""
    if torch is not None and isinstance(x, torch.Tensor):
        return x.detach().to(torch.float64).cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def physical_rows(b: int, L: int, block_table, page_size: int, max_seqlen: int) -> np.ndarray:
    """Cache row of each logical token t in [0, L) of sequence b.

    Paged: the block table maps logical page t // P of sequence b to a pool page.
    Contiguous: sequence b owns rows [b * max_seqlen, b * max_seqlen + L).
    """
    t = np.arange(L, dtype=np.int64)
    if block_table is not None:
        bt = np.asarray(block_table[b] if not hasattr(block_table, "numpy") else block_table[b].numpy(),
                        dtype=np.int64)
        return bt[t // page_size] * page_size + t % page_size
    return b * int(max_seqlen) + t


def rope_scores(q_rope_b: np.ndarray, R: np.ndarray) -> np.ndarray:
    """u[i, t] = <q_rope[i], R[t]>: the RoPE logit of head i, the same for every branch."""
    return q_rope_b @ R.T


def branch_scores(q_j: np.ndarray, C_j: np.ndarray, u: np.ndarray, sm_scale: float) -> np.ndarray:
    """s[i, t] = sm_scale * (<q_j[i], C_j[t]> + u[i, t]) for one latent head (branch) j."""
    return sm_scale * (q_j @ C_j.T + u)


def softmax_average(s: np.ndarray, V: np.ndarray) -> np.ndarray:
    """sum_t softmax(s[i])_t * V[t] per row i (the max is subtracted only for range)."""
    M = s.max(axis=1, keepdims=True)
    w = np.exp(s - M)
    return (w @ V) / w.sum(axis=1, keepdims=True)


def up_project(obar_j: np.ndarray, W_j: np.ndarray) -> np.ndarray:
    """Per head i: the row vector obar_j[i] (D_L) times the matrix W_j[i] (D_L x D_V)."""
    return np.einsum("hc,hcd->hd", obar_j, W_j)


def branch_sum(projected, out_scale: float) -> np.ndarray:
    """out = out_scale * sum over latent heads of the up-projected branch outputs."""
    return out_scale * sum(projected)


def _sequence_operands(q_nope, q_rope, latent, rope, b, L, block_table, page_size, max_seqlen):
    rows = physical_rows(b, L, block_table, page_size, max_seqlen)
    if torch is not None and isinstance(latent, torch.Tensor):
        idx = torch.from_numpy(rows)
        C = as_f64(latent.index_select(0, idx))
        R = as_f64(rope.index_select(0, idx))
    else:
        C = as_f64(np.asarray(latent)[rows])
        R = as_f64(np.asarray(rope)[rows])
    return as_f64(q_nope[b]), as_f64(q_rope[b]), C, R


def decode(q_nope, q_rope, latent, rope, W_UV, seqlens, *, sm_scale: float, out_scale: float,
           block_table=None, page_size: int = 0, max_seqlen: Optional[int] = None,
           batch_indices: Optional[Sequence[int]] = None) -> np.ndarray:
    """Single-pass definition. Shapes: q_nope [B,h,NB,DL], q_rope [B,h,DR],
    latent [rows,NB,DL], rope [rows,DR], W_UV [NB,h,DL,DV], seqlens [B].
    Returns out [len(batch_indices), h, DV] float64 (all sequences by default)."""
    seqlens = [int(x) for x in (seqlens.tolist() if hasattr(seqlens, "tolist") else seqlens)]
    B = len(seqlens)
    NB, h = W_UV.shape[0], W_UV.shape[1]
    DV = W_UV.shape[3]
    if max_seqlen is None:
        max_seqlen = max(seqlens) if seqlens else 0
    W = as_f64(W_UV)
    sel = list(range(B)) if batch_indices is None else list(batch_indices)
    out = np.zeros((len(sel), h, DV), dtype=np.float64)
    for k, b in enumerate(sel):
        L = seqlens[b]
        if L == 0:
            continue
        qn, qr, C, R = _sequence_operands(q_nope, q_rope, latent, rope, b, L, block_table, page_size,
                                          max_seqlen)
        u = rope_scores(qr, R)
        projected = []
        for j in range(NB):
            s = branch_scores(qn[:, j, :], C[:, j, :], u, sm_scale)
            obar = softmax_average(s, C[:, j, :])
            projected.append(up_project(obar, W[j]))
        out[k] = branch_sum(projected, out_scale)
    return out


def partial_stats(s: np.ndarray, V: np.ndarray):
    """Split-KV partial of one chunk: running max m, sum l = sum_t e^{s-m}, O = sum_t e^{s-m} V_t."""
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    return m, e.sum(axis=1), e @ V


def merge_partials(parts):
    """Log-sum-exp merge of chunk partials: obar = sum_c e^{m_c-M} O_c / sum_c e^{m_c-M} l_c."""
    M = np.max(np.stack([p[0] for p in parts]), axis=0)
    num = sum(np.exp(m - M)[:, None] * O for (m, _, O) in parts)
    den = sum(np.exp(m - M) * l for (m, l, _) in parts)
    return num / den[:, None]


def decode_split(q_nope, q_rope, latent, rope, W_UV, seqlens, *, sm_scale: float, out_scale: float,
                 chunk: int, block_table=None, page_size: int = 0,
                 max_seqlen: Optional[int] = None) -> np.ndarray:
    """Split-KV form: each sequence's tokens in chunks of ``chunk``, one partial per chunk,
    merged per (sequence, branch, head). Equal to ``decode`` up to rounding."""
    seqlens = [int(x) for x in (seqlens.tolist() if hasattr(seqlens, "tolist") else seqlens)]
    B = len(seqlens)
    NB, h, DV = W_UV.shape[0], W_UV.shape[1], W_UV.shape[3]
    if max_seqlen is None:
        max_seqlen = max(seqlens) if seqlens else 0
    W = as_f64(W_UV)
    out = np.zeros((B, h, DV), dtype=np.float64)
    for b in range(B):
        L = seqlens[b]
        if L == 0:
            continue
        qn, qr, C, R = _sequence_operands(q_nope, q_rope, latent, rope, b, L, block_table, page_size,
                                          max_seqlen)
        projected = []
        for j in range(NB):
            parts = []
            for t0 in range(0, L, chunk):
                t1 = min(L, t0 + chunk)
                u = rope_scores(qr, R[t0:t1])
                s = branch_scores(qn[:, j, :], C[t0:t1, j, :], u, sm_scale)
                parts.append(partial_stats(s, C[t0:t1, j, :]))
            projected.append(up_project(merge_partials(parts), W[j]))
        out[b] = branch_sum(projected, out_scale)
    return out


def absorb(q_pre, W_UK) -> np.ndarray:
    """Query-side absorption ("Main Findings" bullet 4; block decomposition, "Key
    Contributions" #1): the NoPE key of query head i in latent head j is C_j @ W_UK[j,i]
    (W_UK[j,i] is d_latent x d_nope), so <q_pre, C_j @ W_UK[j,i]> = <W_UK[j,i] @ q_pre, C_j>.
    q_pre [B, h, NB, d_nope], W_UK [NB, h, d_latent, d_nope] -> q_nope [B, h, NB, d_latent]."""
    return np.einsum("jicn,bijn->bijc", as_f64(W_UK), as_f64(q_pre))


def decode_inputs(inp, batch_indices: Optional[Sequence[int]] = None, **overrides) -> np.ndarray:
    """Run ``decode`` on a ``mlra_workloads.DecodeInputs`` bundle (attribute access only)."""
    w = inp.w
    kw = dict(sm_scale=w.sm_scale, out_scale=w.gamma, block_table=inp.block_table,
              page_size=w.page_size, max_seqlen=inp.max_seqlen, batch_indices=batch_indices)
    kw.update(overrides)
    return decode(inp.q_nope, inp.q_rope, inp.latent, inp.rope, inp.W_UV, inp.seqlens, **kw)
