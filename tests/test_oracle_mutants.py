"""Plant one plausible mistake at a time in the oracle (on the CPU) and require the pins to catch it.

This shows the pins are discriminating: a dropped term, a wrong sign or index, a
transposed operand or a merged softmax each fails at least one pin.
"""
import math

import numpy as np
import pytest

import oracle
import oracle_pins
from oracle import mlra_oracle as M


def _mut_rope_dropped(q_rope_b, R):
    return np.zeros((q_rope_b.shape[0], R.shape[0]))


def _mut_rope_sign(q_rope_b, R):
    return -(q_rope_b @ R.T)


def _mut_scale_missing(q_j, C_j, u, sm_scale):
    return q_j @ C_j.T + u


def _mut_scale_nope_only(q_j, C_j, u, sm_scale):
    return sm_scale * (q_j @ C_j.T) + u


def _mut_softmax_wrong_axis(s, V):
    w = np.exp(s - s.max(axis=1, keepdims=True))
    return (w @ V) / w.sum(axis=0, keepdims=True).sum()


def _mut_softmax_no_max(s, V):
    with np.errstate(over="ignore", invalid="ignore"):
        w = np.exp(s)
        return (w @ V) / w.sum(axis=1, keepdims=True)


def _mut_softmax_unnormalised(s, V):
    w = np.exp(s - s.max(axis=1, keepdims=True))
    return w @ V


def _mut_up_transposed(obar_j, W_j):
    return np.einsum("hc,hdc->hd", obar_j, W_j)


def _mut_up_head0(obar_j, W_j):
    return obar_j @ W_j[0]


def _mut_branch_mean(projected, out_scale):
    return out_scale * sum(projected) / len(projected)


def _mut_branch_no_scale(projected, out_scale):
    return sum(projected)


def _mut_rows_swapped(b, L, block_table, page_size, max_seqlen):
    t = np.arange(L, dtype=np.int64)
    if block_table is not None:
        bt = np.asarray(block_table[b], dtype=np.int64)
        return bt[t % page_size] * page_size + t // page_size
    return b * int(max_seqlen) + t


def _mut_rows_ignore_table(b, L, block_table, page_size, max_seqlen):
    return b * int(max_seqlen) + np.arange(L, dtype=np.int64)


def _mut_rows_drop_last(b, L, block_table, page_size, max_seqlen):
    return M.__dict__["_orig_physical_rows"](b, L, block_table, page_size, max_seqlen)[: max(L - 1, 0)]


def _mut_merged_softmax_decode(q_nope, q_rope, latent, rope, W_UV, seqlens, *, sm_scale, out_scale,
                               block_table=None, page_size=0, max_seqlen=None, batch_indices=None):
    """MLA-style: sum the branch logits before one softmax (the block sum kept on K/V)."""
    seqlens = list(seqlens)
    NB, h, DL, DV = W_UV.shape
    out = np.zeros((len(seqlens), h, DV))
    for b, L in enumerate(seqlens):
        if L == 0:
            continue
        rows = M.physical_rows(b, L, block_table, page_size, max_seqlen if max_seqlen else max(seqlens))
        C = np.asarray(latent, dtype=np.float64)[rows]
        R = np.asarray(rope, dtype=np.float64)[rows]
        qn = np.asarray(q_nope[b], dtype=np.float64)
        s = sm_scale * (sum(qn[:, j, :] @ C[:, j, :].T for j in range(NB)) + np.asarray(q_rope[b]) @ R.T)
        w = np.exp(s - s.max(axis=1, keepdims=True))
        w /= w.sum(axis=1, keepdims=True)
        for j in range(NB):
            out[b] += np.einsum("hc,hcd->hd", w @ C[:, j, :], np.asarray(W_UV[j], dtype=np.float64))
        out[b] *= out_scale
    return out


def _mut_rope_first_branch_only_decode(q_nope, q_rope, latent, rope, W_UV, seqlens, *, sm_scale, out_scale,
                                       block_table=None, page_size=0, max_seqlen=None, batch_indices=None):
    seqlens = list(seqlens)
    NB, h, DL, DV = W_UV.shape
    out = np.zeros((len(seqlens), h, DV))
    for b, L in enumerate(seqlens):
        if L == 0:
            continue
        rows = M.physical_rows(b, L, block_table, page_size, max_seqlen if max_seqlen else max(seqlens))
        C = np.asarray(latent, dtype=np.float64)[rows]
        R = np.asarray(rope, dtype=np.float64)[rows]
        u = np.asarray(q_rope[b], dtype=np.float64) @ R.T
        for j in range(NB):
            s = M.branch_scores(np.asarray(q_nope[b][:, j, :], dtype=np.float64), C[:, j, :],
                                u if j == 0 else 0 * u, sm_scale)
            out[b] += M.up_project(M.softmax_average(s, C[:, j, :]), np.asarray(W_UV[j], dtype=np.float64))
        out[b] *= out_scale
    return out


PATCH_MUTANTS = {
    "rope_dropped": ("rope_scores", _mut_rope_dropped),
    "rope_sign": ("rope_scores", _mut_rope_sign),
    "scale_missing": ("branch_scores", _mut_scale_missing),
    "scale_nope_only": ("branch_scores", _mut_scale_nope_only),
    "softmax_wrong_axis": ("softmax_average", _mut_softmax_wrong_axis),
    "softmax_no_max": ("softmax_average", _mut_softmax_no_max),
    "softmax_unnormalised": ("softmax_average", _mut_softmax_unnormalised),
    "up_transposed": ("up_project", _mut_up_transposed),
    "up_head0": ("up_project", _mut_up_head0),
    "branch_mean": ("branch_sum", _mut_branch_mean),
    "branch_no_scale": ("branch_sum", _mut_branch_no_scale),
    "rows_swapped": ("physical_rows", _mut_rows_swapped),
    "rows_ignore_table": ("physical_rows", _mut_rows_ignore_table),
    "rows_drop_last": ("physical_rows", _mut_rows_drop_last),
}

WHOLE_MUTANTS = {
    "merged_softmax": _mut_merged_softmax_decode,
    "rope_first_branch_only": _mut_rope_first_branch_only_decode,
}


def _caught(decode):
    failures = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(decode)
        except Exception as e:  # any error counts as the mutant being caught
            failures.append((pin.__name__, type(e).__name__))
    return failures


@pytest.mark.parametrize("name", sorted(PATCH_MUTANTS))
def test_patched_mutant_is_caught(name, monkeypatch):
    attr, fn = PATCH_MUTANTS[name]
    monkeypatch.setitem(M.__dict__, "_orig_physical_rows", M.physical_rows)
    monkeypatch.setattr(M, attr, fn)
    assert _caught(oracle.decode), f"mutant {name} passed every pin"


@pytest.mark.parametrize("name", sorted(WHOLE_MUTANTS))
def test_whole_mutant_is_caught(name):
    assert _caught(WHOLE_MUTANTS[name]), f"mutant {name} passed every pin"


def test_unmutated_oracle_passes_every_pin():
    assert _caught(oracle.decode) == []


def test_split_merge_mutant_is_caught(monkeypatch):
    """A merge that forgets the e^{m_c - M} weights on the sums breaks split == single pass."""
    def bad_merge(parts):
        num = sum(O for (_, _, O) in parts)
        den = sum(l for (_, l, _) in parts)
        return num / den[:, None]
    monkeypatch.setattr(M, "merge_partials", bad_merge)
    rng = np.random.default_rng(5)
    c = oracle_pins.tiny_case(rng, B=1, h=2, NB=4, DL=3, DR=2, DV=2, Ls=(9,), scale=2.0)
    kw = dict(sm_scale=0.9, out_scale=0.5, max_seqlen=c["max_seqlen"])
    a = oracle.decode(c["q_nope"], c["q_rope"], c["latent"], c["rope"], c["W_UV"], c["seqlens"], **kw)
    s = M.decode_split(c["q_nope"], c["q_rope"], c["latent"], c["rope"], c["W_UV"], c["seqlens"], chunk=4, **kw)
    assert not np.allclose(a, s, rtol=1e-6)


def test_absorb_mutants_are_caught():
    """W_UK of head 0 used for every head, or the query of the wrong latent head, breaks the
    absorption pin."""
    import oracle_pins as P
    bad_head = lambda q_pre, W_UK: np.einsum("jcn,bijn->bijc", np.asarray(W_UK)[:, 0], q_pre)
    bad_branch = lambda q_pre, W_UK: np.einsum("jicn,bijn->bijc", W_UK, np.roll(q_pre, 1, axis=2))
    for bad in (bad_head, bad_branch):
        with pytest.raises(AssertionError):
            P.pin_absorb_is_unabsorbed_attention(oracle.decode, bad)
