"""MLRA-4 / absorbed-MLA single-token decode attention for MI355X (gfx950).

Thin Python binding over libmlra.so (C ABI in include/mlra.h): argument
marshalling only. Every step of the decode runs in the library's HIP kernels;
PyTorch supplies device memory and the current stream. There is no fallback:
if libmlra.so is missing or no GPU is present, calls raise.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib
from ._lib import (MLRA_BF16, MLRA_F32, MLRA_MAX_HEADS, MLRA_NOALLOC_SCRATCH_BYTES, MLRA_TILE_TOKENS, DecodeParams,
                   GqaParams, MlraError, check, lib)

__all__ = ["decode", "decode_splitkv", "decode_combine", "make_params", "Decoder", "workspace_size", "num_splits",
           "check_params", "plan", "copy_bandwidth_probe", "read_bandwidth_probe", "absorb_query", "Absorber", "MlraError",
           "DecodeParams", "GqaParams", "GqaDecoder", "gqa_decode", "make_gqa_params", "MLRA_BF16", "MLRA_F32",
           "MLRA_TILE_TOKENS", "MLRA_MAX_HEADS", "MLRA_NOALLOC_SCRATCH_BYTES", "lib"]

_DTYPES = {torch.bfloat16: MLRA_BF16, torch.float32: MLRA_F32}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def make_params(q_nope: torch.Tensor, q_rope: torch.Tensor, latent_cache: torch.Tensor, rope_cache: torch.Tensor,
                *, sm_scale: float, out_scale: float, max_seqlen: int, page_size: int = 0,
                max_pages_per_seq: int = 0, num_splits: int = 0) -> DecodeParams:
    """Fill the C parameter block from tensor shapes and strides.

    q_nope [B, h, NB, DL], q_rope [B, h, DR], latent_cache [rows, NB, DL], rope_cache [rows, DR]:
    the innermost row of each must be contiguous (views into joint tensors are fine).
    """
    if q_nope.dim() != 4:
        raise ValueError(f"q_nope must be [B, h, NB, d_latent] (got {list(q_nope.shape)})")
    if q_rope.dim() != 3 or latent_cache.dim() != 3 or rope_cache.dim() != 2:
        raise ValueError("q_rope must be [B, h, d_rope], latent_cache [rows, NB, d_latent], rope_cache [rows, d_rope]")
    B, h, NB, DL = q_nope.shape
    if q_nope.stride(3) != 1 or q_nope.stride(2) != DL:
        raise ValueError("q_nope rows [NB, DL] must be contiguous")
    if q_rope.stride(2) != 1 or latent_cache.stride(2) != 1 or latent_cache.stride(1) != DL \
            or rope_cache.stride(1) != 1:
        raise ValueError("q_rope, latent_cache and rope_cache rows must be contiguous")
    if q_nope.dtype not in _DTYPES or any(t.dtype != q_nope.dtype for t in (q_rope, latent_cache, rope_cache)):
        raise ValueError("q_nope, q_rope, latent_cache, rope_cache must share one dtype (bfloat16 or float32)")
    p = DecodeParams()
    p.batch, p.num_heads, p.num_branches, p.d_latent = B, h, NB, DL
    p.d_rope, p.d_v = q_rope.shape[2], 128
    p.dtype = _DTYPES[q_nope.dtype]
    p.page_size, p.max_seqlen, p.max_pages_per_seq, p.num_splits, p.reserved = \
        page_size, max_seqlen, max_pages_per_seq, num_splits, 0
    p.q_stride_b, p.q_stride_h = q_nope.stride(0), q_nope.stride(1)
    p.qr_stride_b, p.qr_stride_h = q_rope.stride(0), q_rope.stride(1)
    p.lat_stride_tok, p.rope_stride_tok = latent_cache.stride(0), rope_cache.stride(0)
    p.sm_scale, p.out_scale = sm_scale, out_scale
    return p


def _same_gpu(tensors, names) -> None:
    """Every tensor given must live on one and the same GPU."""
    devs = {t.device for t in tensors if t is not None}
    bad = [n for t, n in zip(tensors, names) if t is not None and t.device.type != "cuda"]
    if bad:
        raise ValueError(f"{', '.join(bad)} must be GPU tensors")
    if len(devs) > 1:
        raise ValueError(f"{', '.join(names)} must all be on one GPU (got {sorted(str(d) for d in devs)})")


def _check_meta(seqlens, block_table, B: int, paged: bool, max_seqlen: int, page_size: int) -> None:
    if seqlens is None or seqlens.dtype != torch.int32 or not seqlens.is_contiguous() or seqlens.dim() != 1 \
            or seqlens.numel() != B:
        raise ValueError(f"seqlens must be a contiguous int32 tensor of shape [{B}]")
    if paged:
        if block_table is None or block_table.dtype != torch.int32 or not block_table.is_contiguous() \
                or block_table.dim() != 2 or block_table.shape[0] != B:
            raise ValueError(f"block_table must be a contiguous int32 tensor of shape [{B}, max_pages_per_seq]")
        if block_table.shape[1] * page_size < max_seqlen:
            raise ValueError(f"block_table has {block_table.shape[1]} columns of {page_size} tokens, fewer than "
                             f"max_seqlen = {max_seqlen} tokens")
    elif block_table is not None:
        raise ValueError("block_table is given but page_size is 0")


def _check_cache_rows(rows: int, B: int, max_seqlen: int, paged: bool, page_size: int, what: str) -> None:
    """Rows the kernels may address: B * max_seqlen for a contiguous cache; for a paged pool at least one
    page (the block-table entries themselves are device data, which the C ABI leaves unchecked)."""
    if not paged and rows < B * max_seqlen:
        raise ValueError(f"{what} has {rows} rows; a contiguous cache of {B} sequences needs B * max_seqlen = "
                         f"{B * max_seqlen}")
    if paged and B > 0 and rows < page_size:
        raise ValueError(f"{what} has {rows} rows, less than one page of {page_size}")


def _check_decode_tensors(p: DecodeParams, q_nope, q_rope, latent_cache, rope_cache, seqlens, W_UV, block_table,
                          out) -> None:
    """Host-side shape, dtype and layout checks of everything a decode launch reads or writes, so that
    a mismatched tensor raises here instead of sending the kernels out of bounds."""
    B, h, NB, DL = p.batch, p.num_heads, p.num_branches, p.d_latent
    if tuple(q_rope.shape) != (B, h, p.d_rope):
        raise ValueError(f"q_rope must be [{B}, {h}, {p.d_rope}] (got {list(q_rope.shape)})")
    if latent_cache.dim() != 3 or tuple(latent_cache.shape[1:]) != (NB, DL):
        raise ValueError(f"latent_cache must be [rows, {NB}, {DL}] (got {list(latent_cache.shape)})")
    if rope_cache.dim() != 2 or rope_cache.shape[1] != p.d_rope:
        raise ValueError(f"rope_cache must be [rows, {p.d_rope}] (got {list(rope_cache.shape)})")
    if rope_cache.shape[0] != latent_cache.shape[0]:
        raise ValueError(f"latent_cache ({latent_cache.shape[0]} rows) and rope_cache ({rope_cache.shape[0]} rows) "
                         "must share one row numbering")
    paged = p.page_size > 0
    _check_cache_rows(latent_cache.shape[0], B, p.max_seqlen, paged, p.page_size, "latent_cache")
    _check_meta(seqlens, block_table, B, paged, p.max_seqlen, p.page_size)
    if W_UV is None or W_UV.dtype != torch.float32 or not W_UV.is_contiguous() \
            or tuple(W_UV.shape) != (NB, h, DL, p.d_v):
        raise ValueError(f"W_UV must be a contiguous float32 tensor [{NB}, {h}, {DL}, {p.d_v}]"
                         + ("" if W_UV is None else f" (got {W_UV.dtype} {list(W_UV.shape)})"))
    if out is not None and (out.dtype != torch.float32 or not out.is_contiguous()
                            or tuple(out.shape) != (B, h, p.d_v)):
        raise ValueError(f"out must be a contiguous float32 tensor [{B}, {h}, {p.d_v}]")
    _same_gpu((q_nope, q_rope, latent_cache, rope_cache, seqlens, W_UV, block_table, out),
              ("q_nope", "q_rope", "latent_cache", "rope_cache", "seqlens", "W_UV", "block_table", "out"))


def check_params(p: DecodeParams) -> None:
    check(lib().mlra_check_params(ctypes.byref(p)))


def num_splits(p: DecodeParams) -> int:
    n = ctypes.c_int32(0)
    check(lib().mlra_decode_num_splits(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def workspace_size(p: DecodeParams) -> int:
    n = ctypes.c_size_t(0)
    check(lib().mlra_decode_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return n.value


class Decoder:
    """One decode configuration with its workspace, for repeated calls on the same shapes."""

    def __init__(self, q_nope, q_rope, latent_cache, rope_cache, *, seqlens, W_UV, sm_scale, out_scale,
                 max_seqlen, block_table=None, page_size=0, num_splits=0, out=None):
        maxp = 0 if block_table is None else block_table.shape[1]
        self.p = make_params(q_nope, q_rope, latent_cache, rope_cache, sm_scale=sm_scale, out_scale=out_scale,
                             max_seqlen=max_seqlen, page_size=page_size, max_pages_per_seq=maxp,
                             num_splits=num_splits)
        _check_decode_tensors(self.p, q_nope, q_rope, latent_cache, rope_cache, seqlens, W_UV, block_table, out)
        dev = q_nope.device
        self.tensors = (q_nope, q_rope, latent_cache, rope_cache, block_table, seqlens, W_UV)
        self.out = out if out is not None else torch.empty(self.p.batch, self.p.num_heads, 128,
                                                           dtype=torch.float32, device=dev)
        self.ws_bytes = workspace_size(self.p)
        self.workspace = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=dev)
        self.splits = num_splits if num_splits > 0 else self.num_splits()

    def num_splits(self) -> int:
        return num_splits(self.p)

    def __call__(self, stream=None) -> torch.Tensor:
        qn, qr, lat, rp, bt, sl, W = self.tensors
        check(lib().mlra_decode(_ptr(qn), _ptr(qr), _ptr(lat), _ptr(rp), _ptr(bt), _ptr(sl), _ptr(W),
                                _ptr(self.out), ctypes.byref(self.p), _ptr(self.workspace), self.ws_bytes,
                                _stream(stream)))
        return self.out

    def splitkv(self, stream=None) -> None:
        qn, qr, lat, rp, bt, sl, _ = self.tensors
        check(lib().mlra_decode_splitkv(_ptr(qn), _ptr(qr), _ptr(lat), _ptr(rp), _ptr(bt), _ptr(sl),
                                        ctypes.byref(self.p), _ptr(self.workspace), self.ws_bytes, _stream(stream)))

    def capture_graph(self, steps: int = 1) -> "torch.cuda.CUDAGraph":
        """Record `steps` consecutive full decode steps (all kernel launches of mlra_decode) into one
        HIP graph. Replaying it re-runs them on the same tensors; it records kernel launches only.
        The runtime's gap between graph launches is then paid once per `steps` steps."""
        if steps < 1:
            raise ValueError(f"steps must be >= 1 (got {steps})")
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):  # warm-up launch outside the capture
            self(side)
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(steps):
                self()
        return graph

    def combine(self, stream=None) -> torch.Tensor:
        sl, W = self.tensors[5], self.tensors[6]
        check(lib().mlra_decode_combine(_ptr(sl), _ptr(W), _ptr(self.out), ctypes.byref(self.p),
                                        _ptr(self.workspace), self.ws_bytes, _stream(stream)))
        return self.out


def decode(q_nope, q_rope, latent_cache, rope_cache, seqlens, W_UV, *, sm_scale: float, out_scale: float,
           max_seqlen: int, block_table=None, page_size: int = 0, num_splits: int = 0, stream=None) -> torch.Tensor:
    """out[b, i] = out_scale * sum_j softmax-attention of head i over latent head j, up-projected by W_UV[j, i]."""
    return Decoder(q_nope, q_rope, latent_cache, rope_cache, seqlens=seqlens, W_UV=W_UV, sm_scale=sm_scale,
                   out_scale=out_scale, max_seqlen=max_seqlen, block_table=block_table, page_size=page_size,
                   num_splits=num_splits)(stream)


def decode_splitkv(dec: Decoder, stream=None) -> None:
    dec.splitkv(stream)


def decode_combine(dec: Decoder, stream=None) -> torch.Tensor:
    return dec.combine(stream)


def plan(seqlens: torch.Tensor, num_splits: int, max_segments: int, stream=None):
    """The split plan the kernels follow: (segments [G_req, max_segments, 3] int32, total tiles, active splits)."""
    B = seqlens.numel()
    buf = torch.empty(num_splits * max_segments * 3 + 2, dtype=torch.int32, device=seqlens.device)
    check(lib().mlra_decode_plan(_ptr(seqlens), B, num_splits, max_segments, _ptr(buf), _stream(stream)))
    host = buf.cpu()
    segs = host[:-2].view(num_splits, max_segments, 3)
    return segs, int(host[-2]), int(host[-1])


def copy_bandwidth_probe(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst smaller than src")
    check(lib().mlra_copy_bandwidth_probe(_ptr(src), _ptr(dst), nbytes, _stream(stream)))


def read_bandwidth_probe(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """XOR-reduce every 16-byte word of `src` into sink[0] (int32, device)."""
    nbytes = src.numel() * src.element_size()
    check(lib().mlra_read_bandwidth_probe(_ptr(src), nbytes, _ptr(sink), _stream(stream)))


class Absorber:
    """Decode step 1 for fixed tensors: q_nope[b, i, j, :] = W_UK[j, i] @ q_pre[b, i, j, :], written
    into q_nope ([B, h, NB, d_latent], rows contiguous, the layout the decode takes). q_pre is
    [B, h, NB, 128] (a stride-0 branch axis shares one query across latent heads). The C
    arguments are built once; each call is one launch."""

    def __init__(self, q_pre: torch.Tensor, W_UK: torch.Tensor, q_nope: torch.Tensor):
        if q_nope.dim() != 4 or q_pre.dim() != 4 or W_UK.dim() != 4:
            raise ValueError("q_pre must be [B, h, NB, d_nope], W_UK [NB, h, d_latent, d_nope], "
                             "q_nope [B, h, NB, d_latent]")
        B, h, NB, DL = q_nope.shape
        if q_pre.dtype not in _DTYPES or q_nope.dtype != q_pre.dtype:
            raise ValueError("q_pre and q_nope must share one dtype (bfloat16 or float32)")
        if tuple(W_UK.shape) != (NB, h, DL, q_pre.shape[3]):
            raise ValueError(f"W_UK must be [{NB}, {h}, {DL}, {q_pre.shape[3]}] (got {list(W_UK.shape)})")
        if q_pre.shape[:3] != (B, h, NB) or q_pre.stride(3) != 1 or q_pre.dtype != q_nope.dtype:
            raise ValueError("q_pre must be [B, h, NB, d_nope] with contiguous rows and q_nope's dtype")
        if W_UK.dtype != torch.float32 or not W_UK.is_contiguous() or tuple(W_UK.shape[:3]) != (NB, h, DL):
            raise ValueError("W_UK must be a contiguous float32 tensor [NB, h, d_latent, d_nope]")
        if q_nope.stride(3) != 1 or q_nope.stride(2) != DL:
            raise ValueError("q_nope rows [NB, DL] must be contiguous")
        _same_gpu((q_pre, W_UK, q_nope), ("q_pre", "W_UK", "q_nope"))
        p = DecodeParams()
        p.batch, p.num_heads, p.num_branches, p.d_latent, p.d_rope, p.d_v = B, h, NB, DL, 64, 128
        p.dtype = _DTYPES[q_nope.dtype]
        p.q_stride_b, p.q_stride_h = q_nope.stride(0), q_nope.stride(1)
        p.qr_stride_b, p.qr_stride_h = h * 64, 64
        p.lat_stride_tok, p.rope_stride_tok = NB * DL, 64
        p.sm_scale, p.out_scale = 1.0, 1.0
        self.p, self.q_nope = p, q_nope
        self.tensors = (q_pre, W_UK, q_nope)
        self.args = (_ptr(q_pre), _ptr(W_UK), _ptr(q_nope), ctypes.byref(p), q_pre.shape[3], q_pre.stride(0),
                     q_pre.stride(1), q_pre.stride(2))

    def __call__(self, stream=None) -> torch.Tensor:
        check(lib().mlra_absorb_query(*self.args, _stream(stream)))
        return self.q_nope


def absorb_query(q_pre: torch.Tensor, W_UK: torch.Tensor, q_nope: torch.Tensor, stream=None) -> torch.Tensor:
    """Decode step 1 (see Absorber): q_nope[b, i, j, :] = W_UK[j, i] @ q_pre[b, i, j, :]."""
    return Absorber(q_pre, W_UK, q_nope)(stream)


# ---------------------------------------------------------------------------- GQA comparator

def make_gqa_params(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, *, sm_scale: float,
                    max_seqlen: int, page_size: int = 0, max_pages_per_seq: int = 0,
                    num_splits: int = 0) -> GqaParams:
    """q [B, H_q, 128], k_cache / v_cache [rows, H_kv, 128] (bf16; innermost rows contiguous)."""
    if q.dim() != 3 or k_cache.dim() != 3 or v_cache.dim() != 3:
        raise ValueError("q must be [B, H_q, 128], k_cache and v_cache [rows, H_kv, 128]")
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    if k_cache.shape[2] != D or v_cache.shape[2] != D:
        raise ValueError(f"k_cache and v_cache rows must hold {D} channels like q")
    if any(t.dtype != torch.bfloat16 for t in (q, k_cache, v_cache)):
        raise ValueError("q, k_cache and v_cache must be bfloat16")
    if q.stride(2) != 1 or k_cache.stride(2) != 1 or v_cache.stride(2) != 1 or v_cache.shape[1] != Hkv:
        raise ValueError("q, k_cache and v_cache need contiguous head rows and matching KV heads")
    p = GqaParams()
    p.batch, p.num_q_heads, p.num_kv_heads, p.head_dim, p.dtype = B, Hq, Hkv, D, MLRA_BF16
    p.page_size, p.max_seqlen, p.max_pages_per_seq, p.num_splits, p.reserved = \
        page_size, max_seqlen, max_pages_per_seq, num_splits, 0
    p.q_stride_b, p.q_stride_h = q.stride(0), q.stride(1)
    p.k_stride_tok, p.k_stride_head = k_cache.stride(0), k_cache.stride(1)
    p.v_stride_tok, p.v_stride_head = v_cache.stride(0), v_cache.stride(1)
    p.sm_scale, p.reserved_f = sm_scale, 0.0
    return p


class GqaDecoder:
    """One GQA decode configuration with its workspace and output, for repeated calls."""

    def __init__(self, q, k_cache, v_cache, *, seqlens, sm_scale, max_seqlen, block_table=None, page_size=0,
                 num_splits=0):
        maxp = 0 if block_table is None else block_table.shape[1]
        self.p = make_gqa_params(q, k_cache, v_cache, sm_scale=sm_scale, max_seqlen=max_seqlen,
                                 page_size=page_size, max_pages_per_seq=maxp, num_splits=num_splits)
        B = self.p.batch
        if k_cache.dim() != 3 or v_cache.dim() != 3 or k_cache.shape[0] != v_cache.shape[0]:
            raise ValueError("k_cache and v_cache must be [rows, H_kv, 128] with one row numbering")
        _check_cache_rows(k_cache.shape[0], B, max_seqlen, page_size > 0, page_size, "k_cache")
        _check_meta(seqlens, block_table, B, page_size > 0, max_seqlen, page_size)
        _same_gpu((q, k_cache, v_cache, seqlens, block_table), ("q", "k_cache", "v_cache", "seqlens", "block_table"))
        check(lib().mlra_gqa_check_params(ctypes.byref(self.p)))
        self.tensors = (q, k_cache, v_cache, block_table, seqlens)
        self.out = torch.empty(q.shape[0], q.shape[1], q.shape[2], dtype=torch.float32, device=q.device)
        n = ctypes.c_size_t(0)
        check(lib().mlra_gqa_workspace_size(ctypes.byref(self.p), ctypes.byref(n)))
        self.ws_bytes = n.value
        self.workspace = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=q.device)
        g = ctypes.c_int32(0)
        check(lib().mlra_gqa_num_splits(ctypes.byref(self.p), ctypes.byref(g)))
        self.splits = g.value

    def __call__(self, stream=None) -> torch.Tensor:
        q, k, v, bt, sl = self.tensors
        check(lib().mlra_gqa_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(bt), _ptr(sl), _ptr(self.out),
                                    ctypes.byref(self.p), _ptr(self.workspace), self.ws_bytes, _stream(stream)))
        return self.out


def gqa_decode(q, k_cache, v_cache, seqlens, *, sm_scale: float, max_seqlen: int, block_table=None,
               page_size: int = 0, num_splits: int = 0, stream=None) -> torch.Tensor:
    """out[b, i] = softmax_t(sm_scale <q[b,i], K[t, g]>) V[t, g], g = i // (H_q / H_kv)."""
    return GqaDecoder(q, k_cache, v_cache, seqlens=seqlens, sm_scale=sm_scale, max_seqlen=max_seqlen,
                      block_table=block_table, page_size=page_size, num_splits=num_splits)(stream)
