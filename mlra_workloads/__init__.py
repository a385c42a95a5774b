"""Seeded synthetic decode workloads for MLRA-4 and absorbed-MLA decode attention.

This module only draws numbers and lays them out in memory. It holds none of the
method's arithmetic (no logits, no softmax, no projections), so both the fp64 CPU
oracle (``oracle/``) and the HIP path (``long_context_decode_mlra_amd``) can take
their inputs from it without sharing any of the computation.

Shapes follow the MLRA paper's decode setting (Multi-Head Low-Rank Attention,
ai.info summary, "Key Contributions" #2 and "Methodology in Plain English"):
every cached token holds NB latent heads of D_L channels plus one decoupled RoPE
key of D_R = 64 channels; the absorbed query of head i has one D_L-vector per
latent head plus one D_R-vector for the RoPE part. The absorbed MLA comparison
path is NB = 1, D_L = 512, stored as one joint 576-wide row per token.

Draw order for one workload (all from one ``torch.Generator(seed)``):
lengths -> page-pool permutation -> q_nope -> q_rope -> latent -> RoPE -> W_UV.
Every value is an fp32 ``randn`` times the stated standard deviation, cast with
round-to-nearest-even to the storage dtype (W_UV stays fp32).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import torch

__all__ = ["Workload", "WORKLOADS", "make_inputs", "DecodeInputs", "draw_lengths", "make_absorption_inputs",
           "GqaWorkload", "GQA_WORKLOADS", "GqaInputs", "make_gqa_inputs"]

D_ROPE = 64
D_V = 128


@dataclasses.dataclass(frozen=True)
class Workload:
    """One decode workload: shapes, value distributions, layout."""

    name: str
    dtype: str  # "bf16" or "f32": storage of queries and caches
    B: int
    h: int
    NB: int  # latent heads per token (branches): 4 = MLRA-4, 2 = MLRA-2, 1 = MLA
    DL: int  # channels per latent head
    lengths: tuple  # ("fixed", L) | ("uniform", lo, hi) | ("loguniform", lo, hi) | ("list", (L0, L1, ...))
    page_size: int = 0  # 0 = contiguous [B, max_seqlen, ...]; else paged pool
    joint: bool = False  # MLA layout: one [.., NB*DL + DR] row per token for q and cache
    rope_std: float = 1.0
    wuv_std: Optional[float] = None  # default 1/sqrt(DL)
    sm_scale: float = 1.0 / math.sqrt(192.0)
    out_scale: Optional[float] = None  # default 1/sqrt(NB)
    DR: int = D_ROPE
    DV: int = D_V

    @property
    def gamma(self) -> float:
        return self.out_scale if self.out_scale is not None else 1.0 / math.sqrt(self.NB)

    @property
    def w_std(self) -> float:
        return self.wuv_std if self.wuv_std is not None else 1.0 / math.sqrt(self.DL)

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    @property
    def token_elems(self) -> int:
        """Cached elements per token: NB*DL latent + DR RoPE (576 for MLRA-4 and MLA)."""
        return self.NB * self.DL + self.DR

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The workloads of the decode benchmark. Seed = workload number.
WORKLOADS = {
    1: Workload("mlra4_f32_b1_h16_L1k", "f32", B=1, h=16, NB=4, DL=128, lengths=("fixed", 1024)),
    2: Workload("mlra4_bf16_b32_h32_L32k", "bf16", B=32, h=32, NB=4, DL=128, lengths=("fixed", 32768),
                rope_std=math.sqrt(1536.0 / 512.0)),
    3: Workload("mlra4_bf16_b4_h32_L64k-128k", "bf16", B=4, h=32, NB=4, DL=128,
                lengths=("uniform", 65536, 131072)),
    4: Workload("mla_bf16_b32_h32_L32k", "bf16", B=32, h=32, NB=1, DL=512, lengths=("fixed", 32768),
                joint=True),
    5: Workload("mlra4_paged_bf16_b64_h32_L1k-64k", "bf16", B=64, h=32, NB=4, DL=128,
                lengths=("loguniform", 1024, 65536), page_size=64),
    # MLRA-2 (two latent heads of 256 channels, rescale 1/sqrt(2)) at the headline shape.
    6: Workload("mlra2_bf16_b32_h32_L32k", "bf16", B=32, h=32, NB=2, DL=256, lengths=("fixed", 32768)),
    # One GPU's share of workload 2 when its four latent heads are spread over four GPUs: one
    # latent head of 128 channels plus the replicated RoPE keys, one joint 192-wide row per token,
    # the MLRA-4 rescale 1/2 applied before the cross-GPU sum.
    7: Workload("mlra4_shard_bf16_b32_h32_L32k", "bf16", B=32, h=32, NB=1, DL=128, lengths=("fixed", 32768),
                rope_std=math.sqrt(1536.0 / 512.0), out_scale=0.5, joint=True),
}


def draw_lengths(w: Workload, gen: torch.Generator) -> list:
    kind = w.lengths[0]
    if kind == "fixed":
        return [int(w.lengths[1])] * w.B
    if kind == "list":
        Ls = [int(x) for x in w.lengths[1]]
        assert len(Ls) == w.B
        return Ls
    if kind == "uniform":  # integer-uniform, both ends included
        lo, hi = int(w.lengths[1]), int(w.lengths[2])
        return [int(x) for x in torch.randint(lo, hi + 1, (w.B,), generator=gen)]
    if kind == "loguniform":  # floor(exp(U(ln lo, ln hi))), clamped to [lo, hi]
        lo, hi = int(w.lengths[1]), int(w.lengths[2])
        u = torch.rand(w.B, generator=gen, dtype=torch.float64)
        x = torch.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))
        return [min(hi, max(lo, int(math.floor(v)))) for v in x.tolist()]
    raise ValueError(f"unknown length spec {w.lengths!r}")


@dataclasses.dataclass
class DecodeInputs:
    """CPU tensors for one decode step, in the memory layout the library takes.

    Canonical views (always present, possibly strided views of joint tensors):
      q_nope  [B, h, NB, DL]        absorbed NoPE query, one DL-vector per latent head
      q_rope  [B, h, DR]            RoPE part of the query (rotation already applied)
      latent  [rows, NB, DL]        latent cache rows (rows = B*max_seqlen or pages*page_size)
      rope    [rows, DR]            RoPE-key cache rows
      W_UV    [NB, h, DL, DV] fp32  value up-projection per latent head and query head
    plus seqlens [B] int32 and block_table [B, max_pages] int32 (or None).
    For joint (MLA) layouts, ``q_joint`` [B, h, 576] and ``cache_joint`` [rows, 576]
    hold the storage and the canonical tensors are views into them.
    """

    w: Workload
    seqlens: torch.Tensor
    max_seqlen: int
    q_nope: torch.Tensor
    q_rope: torch.Tensor
    latent: torch.Tensor
    rope: torch.Tensor
    W_UV: torch.Tensor
    block_table: Optional[torch.Tensor] = None
    max_pages: int = 0
    q_joint: Optional[torch.Tensor] = None
    cache_joint: Optional[torch.Tensor] = None

    @property
    def paged(self) -> bool:
        return self.block_table is not None

    @property
    def total_tokens(self) -> int:
        return int(self.seqlens.sum())

    def to(self, device) -> "DecodeInputs":
        """Copy every tensor to `device`, keeping joint-layout views as views."""
        mv = lambda t: None if t is None else t.to(device)
        if self.q_joint is not None:
            NB, DL = self.w.NB, self.w.DL
            qj, cj = mv(self.q_joint), mv(self.cache_joint)
            qn, qr = qj[..., :NB * DL].unflatten(-1, (NB, DL)), qj[..., NB * DL:]
            lat, rp = cj[:, :NB * DL].unflatten(-1, (NB, DL)), cj[:, NB * DL:]
        else:
            qj = cj = None
            qn, qr, lat, rp = mv(self.q_nope), mv(self.q_rope), mv(self.latent), mv(self.rope)
        return dataclasses.replace(self, seqlens=mv(self.seqlens), q_nope=qn, q_rope=qr, latent=lat, rope=rp,
                                   W_UV=mv(self.W_UV), block_table=mv(self.block_table), q_joint=qj,
                                   cache_joint=cj)

    def cache_bytes(self) -> int:
        """Bytes of cache one decode step must read: every cached token's latent and RoPE rows."""
        return self.total_tokens * self.w.token_elems * self.w.elem_bytes


def _randn(gen, shape, std, dtype):
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def make_inputs(w: Workload, seed: int, *, lengths: Optional[Sequence[int]] = None,
                poison: bool = False, max_seqlen: Optional[int] = None,
                zero_q_nope: bool = False, zero_q_rope: bool = False) -> DecodeInputs:
    """Draw one workload's tensors on the CPU.

    lengths:   override the length draw (the draw is still consumed first so that the
               stream of later draws does not depend on the override).
    poison:    fill cache rows no sequence owns (contiguous padding, unused page tails)
               with NaN, so that any read of them shows up in the output.
    max_seqlen: contiguous row stride per sequence (default: max length, at least 1).
    """
    gen = torch.Generator().manual_seed(int(seed))
    Ls = draw_lengths(w, gen)
    if lengths is not None:
        Ls = [int(x) for x in lengths]
    B, h, NB, DL, DR = len(Ls), w.h, w.NB, w.DL, w.DR
    dt = w.torch_dtype
    seqlens = torch.tensor(Ls, dtype=torch.int32)
    msl = max(1, max(Ls) if Ls else 1) if max_seqlen is None else int(max_seqlen)
    assert all(L <= msl for L in Ls)

    block_table = None
    max_pages = 0
    if w.page_size:
        P = w.page_size
        pages_per_seq = [(L + P - 1) // P for L in Ls]
        pool = sum(pages_per_seq)
        perm = torch.randperm(max(pool, 1), generator=gen)[:pool]
        max_pages = max(1, (msl + P - 1) // P)
        block_table = torch.full((B, max_pages), -1, dtype=torch.int32)
        off = 0
        for b, n in enumerate(pages_per_seq):
            block_table[b, :n] = perm[off:off + n].to(torch.int32)
            off += n
        rows = max(pool, 1) * P
    else:
        rows = B * msl

    if w.joint:
        q_joint = _randn(gen, (B, h, NB * DL + DR), 1.0, dt)
        if zero_q_nope:
            q_joint[..., :NB * DL] = 0
        if zero_q_rope:
            q_joint[..., NB * DL:] = 0
        cache_joint = _randn(gen, (rows, NB * DL + DR), 1.0, dt)
        if w.rope_std != 1.0:
            cache_joint[:, NB * DL:] = (cache_joint[:, NB * DL:].float() * w.rope_std).to(dt)
        q_nope = q_joint[..., :NB * DL].unflatten(-1, (NB, DL))
        q_rope = q_joint[..., NB * DL:]
        latent = cache_joint[:, :NB * DL].unflatten(-1, (NB, DL))
        rope = cache_joint[:, NB * DL:]
    else:
        q_joint = cache_joint = None
        q_nope = _randn(gen, (B, h, NB, DL), 1.0, dt)
        q_rope = _randn(gen, (B, h, DR), 1.0, dt)
        if zero_q_nope:
            q_nope.zero_()
        if zero_q_rope:
            q_rope.zero_()
        latent = _randn(gen, (rows, NB, DL), 1.0, dt)
        rope = _randn(gen, (rows, DR), w.rope_std, dt)
    W_UV = _randn(gen, (NB, h, DL, w.DV), w.w_std, torch.float32)

    if poison:
        owned = torch.zeros(rows, dtype=torch.bool)
        for b, L in enumerate(Ls):
            if w.page_size:
                P = w.page_size
                t = torch.arange(L)
                pr = block_table[b, (t // P)].long() * P + (t % P)
                owned[pr] = True
            else:
                owned[b * msl: b * msl + L] = True
        bad = ~owned
        if w.joint:
            cache_joint[bad] = float("nan")
        else:
            latent[bad] = float("nan")
            rope[bad] = float("nan")

    return DecodeInputs(w=w, seqlens=seqlens, max_seqlen=msl, q_nope=q_nope, q_rope=q_rope,
                        latent=latent, rope=rope, W_UV=W_UV, block_table=block_table,
                        max_pages=max_pages, q_joint=q_joint, cache_joint=cache_joint)


D_NOPE = 128


def make_absorption_inputs(w: Workload, seed: int, B: int, *, shared_query: bool = False):
    """Pre-absorption NoPE queries and key up-projections for the query-side absorption step.

    From their own generator (seed 1000 * seed + 17), so the workload's other draws are
    unchanged: q_pre [B, h, NB, 128] N(0, 1) in the workload dtype (one vector per head shared
    by every latent head when shared_query: returned as a stride-0 view), then W_UK
    [NB, h, d_latent, 128] fp32 N(0, 1/128)."""
    gen = torch.Generator().manual_seed(1000 * int(seed) + 17)
    if shared_query:
        q = _randn(gen, (B, w.h, 1, D_NOPE), 1.0, w.torch_dtype).expand(B, w.h, w.NB, D_NOPE)
    else:
        q = _randn(gen, (B, w.h, w.NB, D_NOPE), 1.0, w.torch_dtype)
    W_UK = _randn(gen, (w.NB, w.h, w.DL, D_NOPE), 1.0 / math.sqrt(D_NOPE), torch.float32)
    return q, W_UK


# ---------------------------------------------------------------------------- GQA comparator
#
# Grouped-query attention at the shape the MLRA paper analyses it with (ai.info summary,
# "Methodology in Plain English", 4th paragraph: 64 query heads, 8 KV heads, head dim 128):
# the baseline MLRA-4's decode kernel is compared against ("Key Contributions" #4).
# Draw order: lengths -> page-pool permutation -> q -> K cache -> V cache, all N(0, 1).


@dataclasses.dataclass(frozen=True)
class GqaWorkload:
    name: str
    B: int
    Hq: int
    Hkv: int
    lengths: tuple
    page_size: int = 0
    D: int = 128
    dtype: str = "bf16"
    sm_scale: float = 1.0 / math.sqrt(128.0)

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    @property
    def token_elems(self) -> int:
        """Cached elements per token: K and V of every KV head (2048 at H_kv = 8, D = 128)."""
        return 2 * self.Hkv * self.D

    def replace(self, **kw) -> "GqaWorkload":
        return dataclasses.replace(self, **kw)


GQA_WORKLOADS = {
    "gqa_bf16_b32_hq64_hkv8_L32k": GqaWorkload("gqa_bf16_b32_hq64_hkv8_L32k", B=32, Hq=64, Hkv=8,
                                               lengths=("fixed", 32768)),
}


@dataclasses.dataclass
class GqaInputs:
    """q [B, Hq, D], k_cache / v_cache [rows, Hkv, D], seqlens [B] int32, block_table or None."""

    w: GqaWorkload
    seqlens: torch.Tensor
    max_seqlen: int
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_table: Optional[torch.Tensor] = None
    max_pages: int = 0

    @property
    def total_tokens(self) -> int:
        return int(self.seqlens.sum())

    def to(self, device) -> "GqaInputs":
        mv = lambda t: None if t is None else t.to(device)
        return dataclasses.replace(self, seqlens=mv(self.seqlens), q=mv(self.q), k_cache=mv(self.k_cache),
                                   v_cache=mv(self.v_cache), block_table=mv(self.block_table))

    def cache_bytes(self) -> int:
        return self.total_tokens * self.w.token_elems * self.w.elem_bytes


def make_gqa_inputs(w: GqaWorkload, seed: int, *, lengths: Optional[Sequence[int]] = None,
                    poison: bool = False, max_seqlen: Optional[int] = None, zero_q: bool = False,
                    device: str = "cpu") -> GqaInputs:
    """Draw one GQA workload. Lengths and the page permutation always come from a CPU
    generator seeded with `seed`; q, K and V come from the same generator on the CPU, or,
    with device="cuda", from a CUDA generator seeded with 1000 * seed + 29 (a different but
    equally fixed stream, for full-size inputs that are slow to draw on the host)."""
    gen = torch.Generator().manual_seed(int(seed))
    Ls = draw_lengths(w, gen)
    if lengths is not None:
        Ls = [int(x) for x in lengths]
    B, Hq, Hkv, D = len(Ls), w.Hq, w.Hkv, w.D
    seqlens = torch.tensor(Ls, dtype=torch.int32)
    msl = max(1, max(Ls) if Ls else 1) if max_seqlen is None else int(max_seqlen)
    assert all(L <= msl for L in Ls)
    block_table = None
    max_pages = 0
    if w.page_size:
        P = w.page_size
        pages_per_seq = [(L + P - 1) // P for L in Ls]
        pool = sum(pages_per_seq)
        perm = torch.randperm(max(pool, 1), generator=gen)[:pool]
        max_pages = max(1, (msl + P - 1) // P)
        block_table = torch.full((B, max_pages), -1, dtype=torch.int32)
        off = 0
        for b, n in enumerate(pages_per_seq):
            block_table[b, :n] = perm[off:off + n].to(torch.int32)
            off += n
        rows = max(pool, 1) * P
    else:
        rows = B * msl
    if device == "cpu":
        tg, dev = gen, None
    else:
        tg, dev = torch.Generator(device=device).manual_seed(1000 * int(seed) + 29), device
    draw = lambda shape: torch.randn(*shape, generator=tg, dtype=torch.float32, device=dev).to(w.torch_dtype)
    q = draw((B, Hq, D))
    if zero_q:
        q.zero_()
    k_cache = draw((rows, Hkv, D))
    v_cache = draw((rows, Hkv, D))
    if poison:
        owned = torch.zeros(rows, dtype=torch.bool)
        for b, L in enumerate(Ls):
            if w.page_size:
                P = w.page_size
                t = torch.arange(L)
                owned[block_table[b, (t // P)].long() * P + (t % P)] = True
            else:
                owned[b * msl: b * msl + L] = True
        bad = (~owned).to(k_cache.device)
        k_cache[bad] = float("nan")
        v_cache[bad] = float("nan")
    return GqaInputs(w=w, seqlens=seqlens, max_seqlen=msl, q=q, k_cache=k_cache, v_cache=v_cache,
                     block_table=block_table, max_pages=max_pages)
