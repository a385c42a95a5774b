"""Checks that pin the fp64 GQA oracle to facts other than itself.

Each ``pin_*`` takes a callable with the signature of ``oracle.gqa_decode`` and
raises when the callable is wrong. ``test_gqa_oracle.py`` runs them on the
oracle and on copies of it with one planted mistake each.

Sources of truth (GQA as the comparator of the page "Multi-Head Low-Rank
Attention", ai.info summary: "Key Contributions" #4, "Methodology in Plain
English" 4th paragraph):
* a hand-derived golden case (tests/golden/gqa/*.json, exact fractions);
* a pure-Python brute force written from the grouping rule (nested loops,
  math.exp), on tiny inputs;
* a library routine: torch scaled_dot_product_attention in fp64 over K and V
  repeated per query head of each group;
* closed forms: one cached token gives the KV head's value row; a zero query
  gives the mean value row;
* invariants: paged equals contiguous, token order does not matter, a constant
  added to all logits of a head changes nothing (even at logits near 1000), an
  empty sequence gives zero.
"""
from __future__ import annotations

import glob
import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "gqa")


def _arr(x):
    return np.array(json.loads(json.dumps(x).replace("null", "NaN")), dtype=np.float64)


def pin_golden(gqa):
    paths = sorted(glob.glob(os.path.join(GOLDEN_DIR, "*.json")))
    assert paths
    for p in paths:
        d = json.load(open(p))
        sm = math.log(2.0) if d["sm_scale"] == "ln2" else float(Fraction(d["sm_scale"]))
        out = gqa(_arr(d["q"]), _arr(d["k_cache"]), _arr(d["v_cache"]), d["seqlens"], sm_scale=sm,
                  max_seqlen=d["max_seqlen"])
        exp = np.array([[[float(Fraction(v)) for v in row] for row in b] for b in d["expected"]])
        assert np.all(np.isfinite(out)), d["name"]
        np.testing.assert_allclose(out, exp, rtol=1e-13, atol=1e-14, err_msg=d["name"])


def tiny_case(rng, B=2, Hq=6, Hkv=2, D=3, Ls=(5, 3), scale=1.0):
    Ls = list(Ls)
    msl = max(max(Ls), 1)
    return dict(q=rng.normal(size=(B, Hq, D)) * scale, k=rng.normal(size=(B * msl, Hkv, D)),
                v=rng.normal(size=(B * msl, Hkv, D)), seqlens=Ls, max_seqlen=msl)


def pin_bruteforce(gqa):
    rng = np.random.default_rng(11)
    for (Hq, Hkv) in ((6, 2), (4, 4), (5, 1)):
        c = tiny_case(rng, B=2, Hq=Hq, Hkv=Hkv, D=3, Ls=(4, 2), scale=1.3)
        sm = 0.7
        out = gqa(c["q"], c["k"], c["v"], c["seqlens"], sm_scale=sm, max_seqlen=c["max_seqlen"])
        G = Hq // Hkv
        for b, L in enumerate(c["seqlens"]):
            for g in range(Hkv):
                for i in range(g * G, (g + 1) * G):  # the heads of group g
                    logits = []
                    for t in range(L):
                        row = b * c["max_seqlen"] + t
                        logits.append(sm * sum(c["q"][b, i, d] * c["k"][row, g, d] for d in range(3)))
                    mx = max(logits)
                    wts = [math.exp(x - mx) for x in logits]
                    z = sum(wts)
                    for d in range(3):
                        ref = sum(wts[t] * c["v"][b * c["max_seqlen"] + t, g, d] for t in range(L)) / z
                        assert abs(out[b, i, d] - ref) <= 1e-12 * max(1.0, abs(ref)), (Hq, Hkv, b, i, d)


def pin_sdpa_library(gqa):
    rng = np.random.default_rng(12)
    c = tiny_case(rng, B=3, Hq=8, Hkv=2, D=5, Ls=(7, 1, 12), scale=1.1)
    sm = 0.45
    out = gqa(c["q"], c["k"], c["v"], c["seqlens"], sm_scale=sm, max_seqlen=c["max_seqlen"])
    G = 8 // 2
    for b, L in enumerate(c["seqlens"]):
        rows = slice(b * c["max_seqlen"], b * c["max_seqlen"] + L)
        K = torch.from_numpy(c["k"][rows]).permute(1, 0, 2).repeat_interleave(G, dim=0)  # [Hq, L, D]
        V = torch.from_numpy(c["v"][rows]).permute(1, 0, 2).repeat_interleave(G, dim=0)
        Q = torch.from_numpy(c["q"][b]).unsqueeze(1)  # [Hq, 1, D]
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=sm).squeeze(1).numpy()
        np.testing.assert_allclose(out[b], ref, rtol=1e-12, atol=1e-13)


def pin_one_token(gqa):
    rng = np.random.default_rng(13)
    c = tiny_case(rng, B=2, Hq=6, Hkv=3, D=4, Ls=(1, 1))
    out = gqa(c["q"], c["k"], c["v"], c["seqlens"], sm_scale=0.9, max_seqlen=1)
    for b in range(2):
        for i in range(6):
            np.testing.assert_allclose(out[b, i], c["v"][b, i // 2], rtol=1e-14, atol=1e-15)


def pin_zero_query_is_mean(gqa):
    rng = np.random.default_rng(14)
    c = tiny_case(rng, B=2, Hq=4, Hkv=2, D=3, Ls=(6, 3))
    q = np.zeros_like(c["q"])
    out = gqa(q, c["k"], c["v"], c["seqlens"], sm_scale=1.0, max_seqlen=c["max_seqlen"])
    for b, L in enumerate(c["seqlens"]):
        rows = slice(b * c["max_seqlen"], b * c["max_seqlen"] + L)
        for i in range(4):
            np.testing.assert_allclose(out[b, i], c["v"][rows, i // 2].mean(axis=0), rtol=1e-13, atol=1e-14)


def pin_paged_equals_contiguous(gqa):
    rng = np.random.default_rng(15)
    P, Ls = 4, [9, 4, 0, 5]
    c = tiny_case(rng, B=4, Hq=4, Hkv=2, D=3, Ls=Ls)
    msl = c["max_seqlen"]
    ref = gqa(c["q"], c["k"], c["v"], Ls, sm_scale=0.8, max_seqlen=msl)
    pages = [(L + P - 1) // P for L in Ls]
    perm = rng.permutation(sum(pages))
    bt = np.full((4, (msl + P - 1) // P), -1, dtype=np.int64)
    kp = np.full((sum(pages) * P, 2, 3), np.nan)
    vp = np.full_like(kp, np.nan)
    off = 0
    for b, n in enumerate(pages):
        bt[b, :n] = perm[off:off + n]
        off += n
        for t in range(Ls[b]):
            r = bt[b, t // P] * P + t % P
            kp[r] = c["k"][b * msl + t]
            vp[r] = c["v"][b * msl + t]
    out = gqa(c["q"], kp, vp, Ls, sm_scale=0.8, block_table=bt, page_size=P, max_seqlen=msl)
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-14)


def pin_token_permutation(gqa):
    rng = np.random.default_rng(16)
    c = tiny_case(rng, B=1, Hq=4, Hkv=2, D=3, Ls=(8,))
    ref = gqa(c["q"], c["k"], c["v"], c["seqlens"], sm_scale=0.6, max_seqlen=8)
    p = rng.permutation(8)
    out = gqa(c["q"], c["k"][p], c["v"][p], c["seqlens"], sm_scale=0.6, max_seqlen=8)
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-14)


def pin_shift_and_range(gqa):
    """Channel 0 of every key is 1: raising q[..., 0] by s adds sm_scale*s to all logits of that
    head, which leaves its softmax unchanged, up to logits of +-1000."""
    rng = np.random.default_rng(17)
    c = tiny_case(rng, B=2, Hq=4, Hkv=2, D=3, Ls=(6, 4))
    k = c["k"].copy()
    k[:, :, 0] = 1.0
    ref = gqa(c["q"], k, c["v"], c["seqlens"], sm_scale=0.5, max_seqlen=c["max_seqlen"])
    for shift in (2000.0, -2000.0):
        q = c["q"].copy()
        q[..., 0] += shift
        out = gqa(q, k, c["v"], c["seqlens"], sm_scale=0.5, max_seqlen=c["max_seqlen"])
        assert np.all(np.isfinite(out))
        np.testing.assert_allclose(out, ref, rtol=1e-9, atol=1e-10)


def pin_empty_sequence(gqa):
    rng = np.random.default_rng(18)
    c = tiny_case(rng, B=2, Hq=2, Hkv=1, D=3, Ls=(0, 3))
    out = gqa(c["q"], c["k"], c["v"], c["seqlens"], sm_scale=1.0, max_seqlen=c["max_seqlen"])
    assert np.all(out[0] == 0)


ALL_PINS = [pin_golden, pin_bruteforce, pin_sdpa_library, pin_one_token, pin_zero_query_is_mean,
            pin_paged_equals_contiguous, pin_token_permutation, pin_shift_and_range, pin_empty_sequence]
