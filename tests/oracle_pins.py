"""Checks that pin the fp64 oracle to facts other than itself.

Each ``pin_*`` takes a decode callable with the oracle's signature
(``oracle.decode``) and raises AssertionError (or any exception) when the
callable is wrong. ``test_oracle_pins.py`` runs them on the oracle;
``test_oracle_mutants.py`` runs them on copies of the oracle with one planted
mistake each and requires every mistake to be caught.

Sources of truth (page "Multi-Head Low-Rank Attention", ai.info summary):
* hand-derived golden cases (tests/golden/*.json, exact fractions);
* the unabsorbed form: per-head NoPE keys and values materialised from the
  latent by explicit up-projections, which the absorbed form must equal
  ("Main Findings" bullet 4);
* a library routine: per-branch torch scaled_dot_product_attention in fp64
  with K = [C_j, R], V = C_j, then the per-block up-projection and the sum
  ("Key Contributions" #2);
* special cases with closed forms: one cached token, uniform attention,
  q_nope = 0 (all branches share the RoPE-only softmax, so MLRA-4 is exactly
  one half of MLA over the stacked latent: the block decomposition of
  "Key Contributions" #1 and the 1/2 rescale of #3);
* invariants: branch softmaxes are separate (MLRA-4 differs from 1/2 MLA on
  generic data, "Methodology in Plain English" 2nd paragraph), the latent heads
  decoded apart sum to the whole ("Key Contributions" #2), paged equals
  contiguous, token order does not matter, adding a constant to all logits
  of a head does not change its output, an empty sequence gives zero.
"""
from __future__ import annotations

import glob
import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _scalar(sval: str) -> float:
    if sval == "ln2":
        return math.log(2.0)
    return float(Fraction(sval))


def _arr(x):
    """Nested JSON lists to float64; null (a row nobody owns) becomes NaN."""
    return np.array(json.loads(json.dumps(x).replace("null", "NaN")), dtype=np.float64)


def load_golden(path):
    d = json.load(open(path))
    bt = d.get("block_table")
    return dict(
        name=d["name"],
        q_nope=_arr(d["q_nope"]), q_rope=_arr(d["q_rope"]), latent=_arr(d["latent"]), rope=_arr(d["rope"]),
        W_UV=_arr(d["W_UV"]), seqlens=d["seqlens"],
        kw=dict(sm_scale=_scalar(d["sm_scale"]), out_scale=_scalar(d["out_scale"]),
                block_table=None if bt is None else np.array(bt, dtype=np.int64),
                page_size=d["page_size"], max_seqlen=d["max_seqlen"]),
        expected=np.array([[[float(Fraction(v)) for v in row] for row in head] for head in d["expected"]]),
    )


def golden_paths():
    return sorted(glob.glob(os.path.join(GOLDEN_DIR, "*.json")))


def pin_golden(decode):
    for p in golden_paths():
        g = load_golden(p)
        out = decode(g["q_nope"], g["q_rope"], g["latent"], g["rope"], g["W_UV"], g["seqlens"], **g["kw"])
        assert np.all(np.isfinite(out)), g["name"]
        np.testing.assert_allclose(out, g["expected"], rtol=1e-13, atol=1e-14, err_msg=g["name"])


# ---------------------------------------------------------------- random tiny inputs
def tiny_case(rng, B=2, h=3, NB=4, DL=4, DR=2, DV=3, Ls=(5, 3), scale=1.0):
    Ls = list(Ls)
    msl = max(Ls)
    return dict(
        q_nope=rng.standard_normal((B, h, NB, DL)) * scale,
        q_rope=rng.standard_normal((B, h, DR)) * scale,
        latent=rng.standard_normal((B * msl, NB, DL)),
        rope=rng.standard_normal((B * msl, DR)),
        W_UV=rng.standard_normal((NB, h, DL, DV)),
        seqlens=Ls, max_seqlen=msl,
    )


def _call(decode, c, **kw):
    args = dict(sm_scale=kw.pop("sm_scale", 0.37), out_scale=kw.pop("out_scale", 1.0 / math.sqrt(c["W_UV"].shape[0])),
                max_seqlen=c["max_seqlen"])
    args.update(kw)
    return decode(c["q_nope"], c["q_rope"], c["latent"], c["rope"], c["W_UV"], c["seqlens"], **args)


def pin_unabsorbed_bruteforce(decode):
    """Absorbed decode == attention with explicit per-head NoPE keys/values (pure Python loops)."""
    rng = np.random.default_rng(11)
    for (NB, Ls) in ((4, (5, 1, 3)), (1, (4, 2, 0)), (2, (6, 2, 1))):
        B, h, DL, DR, DV, dn = len(Ls), 3, 4, 2, 3, 5
        msl = max(Ls)
        q_pre = rng.standard_normal((B, h, NB, dn))
        W_UK = rng.standard_normal((NB, h, DL, dn))  # latent (DL) -> per-head NoPE key (dn)
        q_rope = rng.standard_normal((B, h, DR))
        lat = rng.standard_normal((B * msl, NB, DL))
        rope = rng.standard_normal((B * msl, DR))
        W_UV = rng.standard_normal((NB, h, DL, DV))
        sm, gam = 0.41, 1.0 / math.sqrt(NB)
        expect = np.zeros((B, h, DV))
        for b in range(B):
            L = Ls[b]
            for i in range(h):
                acc = [0.0] * DV
                for j in range(NB):
                    logits, vals = [], []
                    for t in range(L):
                        row = b * msl + t
                        k = [sum(lat[row, j, c] * W_UK[j, i, c, e] for c in range(DL)) for e in range(dn)]
                        v = [sum(lat[row, j, c] * W_UV[j, i, c, d] for c in range(DL)) for d in range(DV)]
                        nope = sum(q_pre[b, i, j, e] * k[e] for e in range(dn))
                        rp = sum(q_rope[b, i, r] * rope[row, r] for r in range(DR))
                        logits.append(sm * (nope + rp))
                        vals.append(v)
                    if L == 0:
                        continue
                    mx = max(logits)
                    ws = [math.exp(x - mx) for x in logits]
                    Z = sum(ws)
                    for d in range(DV):
                        acc[d] += sum(ws[t] * vals[t][d] for t in range(L)) / Z
                expect[b, i] = [gam * a for a in acc]
        # absorb: q_nope[b,i,j,c] = sum_e W_UK[j,i,c,e] q_pre[b,i,j,e]
        q_nope = np.zeros((B, h, NB, DL))
        for b in range(B):
            for i in range(h):
                for j in range(NB):
                    for c in range(DL):
                        q_nope[b, i, j, c] = sum(W_UK[j, i, c, e] * q_pre[b, i, j, e] for e in range(dn))
        got = decode(q_nope, q_rope, lat, rope, W_UV, list(Ls), sm_scale=sm, out_scale=gam, max_seqlen=msl)
        np.testing.assert_allclose(got, expect, rtol=1e-11, atol=1e-12)


def pin_sdpa_library(decode):
    """Per-branch torch SDPA (fp64, K=[C_j,R], V=C_j) at the real widths, then W_UV blocks summed."""
    rng = np.random.default_rng(12)
    for (NB, DL) in ((4, 128), (1, 512)):
        B, h, DR, DV = 2, 8, 64, 128
        Ls = (300, 77)
        c = tiny_case(rng, B=B, h=h, NB=NB, DL=DL, DR=DR, DV=DV, Ls=Ls)
        sm, gam = 1.0 / math.sqrt(192.0), 1.0 / math.sqrt(NB)
        got = _call(decode, c, sm_scale=sm, out_scale=gam)
        W = torch.from_numpy(c["W_UV"])
        for b in range(B):
            L = Ls[b]
            rows = torch.arange(b * c["max_seqlen"], b * c["max_seqlen"] + L)
            C = torch.from_numpy(c["latent"])[rows]  # [L, NB, DL]
            R = torch.from_numpy(c["rope"])[rows]    # [L, DR]
            acc = torch.zeros(h, DV, dtype=torch.float64)
            for j in range(NB):
                Q = torch.cat([torch.from_numpy(c["q_nope"][b, :, j, :]), torch.from_numpy(c["q_rope"][b])], -1)
                K = torch.cat([C[:, j, :], R], -1)
                o = torch.nn.functional.scaled_dot_product_attention(
                    Q[None, :, None, :], K[None, None].expand(1, h, L, DL + DR).contiguous(),
                    C[None, None, :, j, :].expand(1, h, L, DL).contiguous(), scale=sm)[0, :, 0, :]  # [h, DL]
                acc += torch.bmm(o[:, None, :], W[j].contiguous())[:, 0, :]
            np.testing.assert_allclose(got[b], (gam * acc).numpy(), rtol=1e-10, atol=1e-12)


def pin_shared_rope_half_mla(decode):
    """q_nope = 0: every branch has the same RoPE-only softmax, so MLRA-4 (gamma 1/2) equals
    1/2 of MLA (gamma 1) over the stacked latent with the stacked W_UV blocks (exact)."""
    rng = np.random.default_rng(13)
    c = tiny_case(rng, B=2, h=3, NB=4, DL=4, DR=3, DV=2, Ls=(6, 4))
    c["q_nope"][:] = 0.0
    mlra = _call(decode, c, sm_scale=0.9, out_scale=0.5)
    B, h, NB, DL = c["q_nope"].shape
    mla = decode(np.zeros((B, h, 1, NB * DL)), c["q_rope"], c["latent"].reshape(-1, 1, NB * DL), c["rope"],
                 c["W_UV"].transpose(1, 0, 2, 3).reshape(1, h, NB * DL, -1), c["seqlens"], sm_scale=0.9,
                 out_scale=1.0, max_seqlen=c["max_seqlen"])
    np.testing.assert_allclose(mlra, 0.5 * mla, rtol=1e-12, atol=1e-13)


def pin_shards_sum_to_whole(decode):
    """The latent heads can be decoded apart (one per GPU in the pages' tensor-parallel layout,
    "Key Contributions" #2): decoding each latent head alone, with its own W_UV block and the
    same rescale, and summing the NB results gives the NB-head output (exact)."""
    rng = np.random.default_rng(16)
    c = tiny_case(rng, B=2, h=3, NB=4, DL=4, DR=3, DV=2, Ls=(9, 3), scale=1.5)
    whole = _call(decode, c, sm_scale=0.7, out_scale=0.5)
    parts = [decode(c["q_nope"][:, :, j:j + 1], c["q_rope"], c["latent"][:, j:j + 1], c["rope"],
                    c["W_UV"][j:j + 1], c["seqlens"], sm_scale=0.7, out_scale=0.5, max_seqlen=c["max_seqlen"])
             for j in range(4)]
    np.testing.assert_allclose(sum(parts), whole, rtol=1e-12, atol=1e-13)


def pin_branches_separate(decode):
    """Generic q_nope: per-branch softmaxes are not the MLA softmax; the results must differ."""
    rng = np.random.default_rng(14)
    c = tiny_case(rng, B=1, h=2, NB=4, DL=4, DR=2, DV=2, Ls=(7,), scale=2.0)
    mlra = _call(decode, c, sm_scale=0.8, out_scale=0.5)
    B, h, NB, DL = c["q_nope"].shape
    mla = decode(c["q_nope"].reshape(B, h, 1, NB * DL), c["q_rope"], c["latent"].reshape(-1, 1, NB * DL),
                 c["rope"], c["W_UV"].transpose(1, 0, 2, 3).reshape(1, h, NB * DL, -1), c["seqlens"],
                 sm_scale=0.8, out_scale=1.0, max_seqlen=c["max_seqlen"])
    rel = np.linalg.norm(mlra - 0.5 * mla) / np.linalg.norm(mlra)
    assert rel > 1e-2, rel


def pin_one_token(decode):
    """L = 1: softmax of one logit is 1, so out = gamma * sum_j C_0j @ W_UV[j, i]."""
    rng = np.random.default_rng(15)
    c = tiny_case(rng, B=3, h=2, NB=4, DL=3, DR=2, DV=4, Ls=(1, 1, 1))
    got = _call(decode, c, sm_scale=1.3, out_scale=0.5)
    for b in range(3):
        C = c["latent"][b * c["max_seqlen"]]
        exp = np.stack([0.5 * sum(C[j] @ c["W_UV"][j, i] for j in range(4)) for i in range(2)])
        np.testing.assert_allclose(got[b], exp, rtol=1e-13, atol=1e-14)


def pin_uniform(decode):
    """q_nope = 0 and q_rope = 0: uniform weights, obar_j = mean_t C_tj."""
    rng = np.random.default_rng(16)
    c = tiny_case(rng, B=2, h=2, NB=4, DL=3, DR=2, DV=2, Ls=(5, 2))
    c["q_nope"][:] = 0
    c["q_rope"][:] = 0
    got = _call(decode, c, sm_scale=0.7, out_scale=0.5)
    for b, L in enumerate(c["seqlens"]):
        C = c["latent"][b * c["max_seqlen"]: b * c["max_seqlen"] + L]
        mean = C.mean(axis=0)  # [NB, DL]
        exp = np.stack([0.5 * sum(mean[j] @ c["W_UV"][j, i] for j in range(4)) for i in range(2)])
        np.testing.assert_allclose(got[b], exp, rtol=1e-13, atol=1e-14)


def pin_paged_equals_contiguous(decode):
    """A permuted page pool read through the block table gives the contiguous result."""
    rng = np.random.default_rng(17)
    P = 4
    Ls = [9, 0, 4, 13]
    c = tiny_case(rng, B=4, h=2, NB=4, DL=3, DR=2, DV=2, Ls=Ls)
    cont = _call(decode, c)
    pages = [(L + P - 1) // P for L in Ls]
    perm = rng.permutation(sum(pages))
    maxp = max(pages)
    bt = -np.ones((4, maxp), dtype=np.int64)
    lat = np.full((sum(pages) * P, 4, 3), np.nan)
    rp = np.full((sum(pages) * P, 2), np.nan)
    off = 0
    for b, L in enumerate(Ls):
        for p in range(pages[b]):
            bt[b, p] = perm[off + p]
        for t in range(L):
            row = bt[b, t // P] * P + t % P
            lat[row] = c["latent"][b * c["max_seqlen"] + t]
            rp[row] = c["rope"][b * c["max_seqlen"] + t]
        off += pages[b]
    paged = decode(c["q_nope"], c["q_rope"], lat, rp, c["W_UV"], Ls, sm_scale=0.37, out_scale=0.5,
                   block_table=bt, page_size=P, max_seqlen=maxp * P)
    np.testing.assert_allclose(paged, cont, rtol=1e-13, atol=1e-14)


def pin_token_permutation(decode):
    """Attention is a set function of the cached tokens: permuting them changes nothing."""
    rng = np.random.default_rng(18)
    c = tiny_case(rng, B=1, h=2, NB=4, DL=3, DR=2, DV=2, Ls=(8,))
    a = _call(decode, c)
    perm = rng.permutation(8)
    c2 = dict(c)
    c2["latent"] = c["latent"][perm]
    c2["rope"] = c["rope"][perm]
    np.testing.assert_allclose(_call(decode, c2), a, rtol=1e-13, atol=1e-14)


def pin_shift_and_range(decode):
    """A constant added to every logit of a head leaves its output unchanged, even when the
    constant is far outside fp64 exp's range (logits +-1000 through an extra RoPE channel)."""
    rng = np.random.default_rng(19)
    c = tiny_case(rng, B=1, h=2, NB=4, DL=3, DR=3, DV=2, Ls=(6,))
    c["q_rope"][..., 2] = 0.0
    c["rope"][:, 2] = 1.0
    base = _call(decode, c, sm_scale=0.5)
    for shift in (2000.0, -2000.0):  # times sm_scale 0.5
        c2 = dict(c)
        c2["q_rope"] = c["q_rope"].copy()
        c2["q_rope"][..., 2] = shift
        got = _call(decode, c2, sm_scale=0.5)
        assert np.all(np.isfinite(got))
        np.testing.assert_allclose(got, base, rtol=1e-10, atol=1e-12)


def pin_empty_sequence(decode):
    rng = np.random.default_rng(20)
    c = tiny_case(rng, B=3, h=2, NB=4, DL=3, DR=2, DV=2, Ls=(0, 3, 0))
    got = _call(decode, c)
    assert np.all(got[0] == 0) and np.all(got[2] == 0)
    assert np.all(np.isfinite(got[1])) and np.any(got[1] != 0)


def pin_absorb_is_unabsorbed_attention(decode, absorb=None):
    """decode(absorb(q_pre, W_UK)) equals attention with the per-head NoPE keys C_j @ W_UK[j,i]
    materialised and dotted with q_pre directly (no absorption anywhere on this side)."""
    import oracle
    absorb = absorb or oracle.absorb
    rng = np.random.default_rng(21)
    for NB in (4, 1):
        B, h, DL, DR, DV, dn, Ls = 2, 3, 4 if NB == 4 else 8, 2, 3, 5, (6, 3)
        msl = max(Ls)
        q_pre = rng.standard_normal((B, h, NB, dn))
        W_UK = rng.standard_normal((NB, h, DL, dn))
        q_rope = rng.standard_normal((B, h, DR))
        lat = rng.standard_normal((B * msl, NB, DL))
        rope = rng.standard_normal((B * msl, DR))
        W_UV = rng.standard_normal((NB, h, DL, DV))
        got = decode(absorb(q_pre, W_UK), q_rope, lat, rope, W_UV, list(Ls), sm_scale=0.3,
                     out_scale=1 / math.sqrt(NB), max_seqlen=msl)
        for b in range(B):
            rows = np.arange(b * msl, b * msl + Ls[b])
            for i in range(h):
                acc = np.zeros(DV)
                for j in range(NB):
                    K = lat[rows, j, :] @ W_UK[j, i]                    # [L, dn] NoPE keys
                    logit = 0.3 * (K @ q_pre[b, i, j] + rope[rows] @ q_rope[b, i])
                    p = np.exp(logit - logit.max())
                    p /= p.sum()
                    acc += (p @ lat[rows, j, :]) @ W_UV[j, i]           # values then up-projection
                np.testing.assert_allclose(got[b, i], acc / math.sqrt(NB), rtol=1e-11, atol=1e-12)


ALL_PINS = [pin_golden, pin_unabsorbed_bruteforce, pin_sdpa_library, pin_shared_rope_half_mla,
            pin_shards_sum_to_whole, pin_branches_separate, pin_one_token, pin_uniform, pin_paged_equals_contiguous,
            pin_token_permutation, pin_shift_and_range, pin_empty_sequence, pin_absorb_is_unabsorbed_attention]
