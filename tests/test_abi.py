"""The C ABI on the CPU: the library loads, exports every declared symbol, and the
host-only validation rejects each kind of bad argument (no GPU needed, no kernel runs)."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    from long_context_decode_mlra_amd import _lib as L
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("libmlra.so not built (run __graft_entry__.build())")
    return L


def test_header_declares_exactly_the_exported_symbols():
    L = _lib()
    header = open(os.path.join(ROOT, "include", "mlra.h")).read()
    declared = set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(mlra_\w+)\s*\(", header, re.M))
    assert declared == set(L.EXPORTS)
    lib = L.lib()
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.mlra_abi_version() == 1


def test_exports_visible_to_dynamic_loader():
    L = _lib()
    raw = ctypes.CDLL(L.LIB_PATH)
    for name in L.EXPORTS:
        assert ctypes.cast(getattr(raw, name), ctypes.c_void_p).value


def good_params(**kw):
    L = _lib()
    p = L.DecodeParams()
    p.batch, p.num_heads, p.num_branches, p.d_latent, p.d_rope, p.d_v = 32, 32, 4, 128, 64, 128
    p.dtype, p.page_size, p.max_seqlen, p.max_pages_per_seq, p.num_splits, p.reserved = 0, 0, 32768, 0, 512, 0
    p.q_stride_b, p.q_stride_h, p.qr_stride_b, p.qr_stride_h = 32 * 512, 512, 32 * 64, 64
    p.lat_stride_tok, p.rope_stride_tok = 512, 64
    p.sm_scale, p.out_scale = 1 / math.sqrt(192), 0.5
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def rc(p):
    L = _lib()
    return L.lib().mlra_check_params(ctypes.byref(p))


def test_valid_params_pass():
    assert rc(good_params()) == 0
    assert rc(good_params(num_branches=1, d_latent=512, q_stride_h=576, lat_stride_tok=576,
                          rope_stride_tok=576, qr_stride_h=576, qr_stride_b=32 * 576, q_stride_b=32 * 576)) == 0
    assert rc(good_params(num_branches=2, d_latent=256)) == 0
    assert rc(good_params(dtype=1, num_heads=16)) == 0
    assert rc(good_params(page_size=64, max_pages_per_seq=512)) == 0
    assert rc(good_params(batch=0)) == 0


@pytest.mark.parametrize("field,value,code", [
    ("num_heads", 0, -3), ("num_heads", 65, -3), ("num_branches", 3, -3), ("d_latent", 64, -3),
    ("d_rope", 32, -3), ("d_v", 64, -3), ("dtype", 7, -3), ("batch", -1, -2), ("max_seqlen", -5, -2),
    ("page_size", 48, -3), ("page_size", -64, -2), ("num_splits", -1, -2), ("reserved", 1, -2),
    ("q_stride_h", 100, -2), ("lat_stride_tok", 500, -2), ("rope_stride_tok", 63, -2),
    ("q_stride_h", 516, -4), ("lat_stride_tok", 516, -4), ("qr_stride_b", 2052, -4),
    ("sm_scale", 0.0, -2), ("sm_scale", float("nan"), -2), ("out_scale", float("inf"), -2),
    ("lat_stride_tok", 1 << 25, -2),
])
def test_bad_params_rejected(field, value, code):
    assert rc(good_params(**{field: value})) == code
    L = _lib()
    assert L.lib().mlra_last_error().decode()


def shard_params(**kw):
    """One latent head of 128 channels plus RoPE in joint 192-element rows (the shard form)."""
    base = dict(num_branches=1, d_latent=128, q_stride_b=32 * 192, q_stride_h=192, qr_stride_b=32 * 192,
                qr_stride_h=192, lat_stride_tok=192, rope_stride_tok=192)
    base.update(kw)
    return good_params(**base)


def test_shard_form_params():
    assert rc(shard_params()) == 0
    assert rc(shard_params(num_heads=1)) == 0
    assert rc(shard_params(page_size=64, max_pages_per_seq=512)) == 0
    assert rc(shard_params(dtype=1)) == -3          # bf16 only
    assert rc(shard_params(num_heads=33)) == -3     # one block of 32 query heads
    assert rc(shard_params(num_branches=2)) == -3   # 2 x 128 is not a supported latent
    assert rc(shard_params(q_stride_h=120)) == -2   # below the 128-element latent row


def test_shard_workspace_size_with_explicit_splits_needs_no_device():
    L = _lib()
    p = shard_params(num_splits=1024)
    n = ctypes.c_size_t(0)
    assert L.lib().mlra_decode_workspace_size(ctypes.byref(p), ctypes.byref(n)) == 0
    slots = 1024 + 32
    expect = (slots * 32 * 128 * 2          # split partials of the output (one latent head), fp16
              + slots * 32 * 2 * 4          # one exponent per 64-channel block of each partial
              + slots * 1 * 32 * 2 * 4      # running max and sum per partial
              + (32 + 3) * 8                # tile prefix per sequence, T, G
              + 1 * 32 * 2 * 32 * 128 * 4   # projected 64-channel blocks, one group of 32 sequences
              + 32 * 8 * 4)                 # combine arrival counters
    assert n.value >= expect and n.value % 256 == 0 and n.value < expect + 6 * 256


def test_paged_needs_enough_table_columns():
    assert rc(good_params(page_size=64, max_pages_per_seq=511)) == -2
    assert rc(good_params(page_size=64, max_pages_per_seq=512)) == 0


def test_null_params():
    L = _lib()
    assert L.lib().mlra_check_params(None) == -1


def test_workspace_size_with_explicit_splits_needs_no_device():
    L = _lib()
    p = good_params(num_splits=512)
    n = ctypes.c_size_t(0)
    assert L.lib().mlra_decode_workspace_size(ctypes.byref(p), ctypes.byref(n)) == 0
    slots = 512 + 32
    for dtype, esz, exps in ((0, 2, 8 * 4), (1, 4, 0)):  # bf16: fp16 partials + block exponents; fp32
        p = good_params(num_splits=512, dtype=dtype)
        assert L.lib().mlra_decode_workspace_size(ctypes.byref(p), ctypes.byref(n)) == 0
        expect = (slots * 32 * 512 * esz        # split partials of the output
                  + slots * 32 * exps           # one exponent per 64-channel block (bf16 only)
                  + slots * 4 * 32 * 2 * 4      # running max and sum per partial
                  + (32 + 3) * 8                # tile prefix per sequence, T, G
                  + 1 * 32 * 8 * 32 * 128 * 4   # projected 64-channel blocks, one group of 32 sequences
                  + 32 * 8 * 4)                 # combine arrival counters
        assert n.value >= expect and n.value % 256 == 0 and n.value < expect + 6 * 256, dtype


def test_decode_argument_errors_before_any_launch():
    """Pointer and workspace checks happen on the host before any HIP call."""
    L = _lib()
    lib = L.lib()
    p = good_params(num_splits=8)
    fake = ctypes.c_void_p(1 << 20)
    # workspace too small
    r = lib.mlra_decode(fake, fake, fake, fake, None, fake, fake, fake, ctypes.byref(p), fake, 256, None)
    assert r == -5
    # NULL query pointer
    n = ctypes.c_size_t(0)
    lib.mlra_decode_workspace_size(ctypes.byref(p), ctypes.byref(n))
    r = lib.mlra_decode(None, fake, fake, fake, None, fake, fake, fake, ctypes.byref(p), fake, n.value, None)
    assert r == -1
    # misaligned cache pointer
    r = lib.mlra_decode(fake, fake, ctypes.c_void_p((1 << 20) + 8), fake, None, fake, fake, fake, ctypes.byref(p),
                        fake, n.value, None)
    assert r == -4
    # block_table given for a contiguous cache
    r = lib.mlra_decode(fake, fake, fake, fake, fake, fake, fake, fake, ctypes.byref(p), fake, n.value, None)
    assert r == -1
    # misaligned workspace
    r = lib.mlra_decode(fake, fake, fake, fake, None, fake, fake, fake, ctypes.byref(p),
                        ctypes.c_void_p((1 << 20) + 16), n.value, None)
    assert r == -4
    # misaligned output
    r = lib.mlra_decode(fake, fake, fake, fake, None, fake, fake, ctypes.c_void_p((1 << 20) + 4), ctypes.byref(p),
                        fake, n.value, None)
    assert r == -4
    assert lib.mlra_decode_plan(fake, 4, 0, 4, fake, None) == -2
    assert lib.mlra_copy_bandwidth_probe(fake, ctypes.c_void_p((1 << 20) + 4), 64, None) == -4


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    from long_context_decode_mlra_amd import _lib as L
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(L, "_lib", None)
    with pytest.raises(ImportError):
        L.lib()


# ---------------------------------------------------------------------------- GQA comparator
def good_gqa(**kw):
    L = _lib()
    p = L.GqaParams()
    p.batch, p.num_q_heads, p.num_kv_heads, p.head_dim, p.dtype = 32, 64, 8, 128, 0
    p.page_size, p.max_seqlen, p.max_pages_per_seq, p.num_splits, p.reserved = 0, 32768, 0, 96, 0
    p.q_stride_b, p.q_stride_h = 64 * 128, 128
    p.k_stride_tok, p.k_stride_head, p.v_stride_tok, p.v_stride_head = 8 * 128, 128, 8 * 128, 128
    p.sm_scale, p.reserved_f = 1 / math.sqrt(128), 0.0
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def gqa_rc(p):
    return _lib().lib().mlra_gqa_check_params(ctypes.byref(p))


def test_gqa_valid_params_pass():
    assert gqa_rc(good_gqa()) == 0
    assert gqa_rc(good_gqa(num_q_heads=16, num_kv_heads=1)) == 0
    assert gqa_rc(good_gqa(page_size=64, max_pages_per_seq=512)) == 0


@pytest.mark.parametrize("field,value,code", [
    ("batch", -1, -2), ("num_kv_heads", 0, -2), ("num_q_heads", 60, -2), ("num_q_heads", 136, -3),
    ("head_dim", 64, -3), ("dtype", 1, -3), ("max_seqlen", -1, -2), ("page_size", 48, -3),
    ("page_size", 64, -2), ("num_splits", -1, -2), ("reserved", 1, -2), ("reserved_f", 1.0, -2),
    ("q_stride_h", 64, -2), ("k_stride_tok", -8, -2), ("v_stride_head", 100, -4), ("q_stride_b", 8 * 128 + 4, -4),
    ("k_stride_tok", 1 << 25, -2), ("sm_scale", 0.0, -2), ("sm_scale", float("inf"), -2),
])
def test_gqa_bad_params_rejected(field, value, code):
    assert gqa_rc(good_gqa(**{field: value})) == code


def test_gqa_workspace_size_with_explicit_splits_needs_no_device():
    L = _lib()
    p = good_gqa(num_splits=96)
    n = ctypes.c_size_t(0)
    assert L.lib().mlra_gqa_workspace_size(ctypes.byref(p), ctypes.byref(n)) == 0
    slots = 96 + 32
    expect = slots * 64 * 128 * 4 + slots * 64 * 2 * 4 + 35 * 8
    assert n.value >= expect and n.value % 256 == 0 and n.value < expect + 3 * 256


def test_gqa_argument_errors_before_any_launch():
    L = _lib()
    lib = L.lib()
    p = good_gqa(num_splits=8)
    fake = ctypes.c_void_p(1 << 20)
    n = ctypes.c_size_t(0)
    lib.mlra_gqa_workspace_size(ctypes.byref(p), ctypes.byref(n))
    assert lib.mlra_gqa_decode(fake, fake, fake, None, fake, fake, ctypes.byref(p), fake, 256, None) == -5
    assert lib.mlra_gqa_decode(None, fake, fake, None, fake, fake, ctypes.byref(p), fake, n.value, None) == -1
    assert lib.mlra_gqa_decode(fake, ctypes.c_void_p((1 << 20) + 8), fake, None, fake, fake, ctypes.byref(p), fake,
                               n.value, None) == -4
    assert lib.mlra_gqa_decode(fake, fake, fake, fake, fake, fake, ctypes.byref(p), fake, n.value, None) == -1
    assert lib.mlra_gqa_decode(fake, fake, fake, None, None, fake, ctypes.byref(p), fake, n.value, None) == -1


def test_absorb_argument_errors_before_any_launch():
    L = _lib()
    lib = L.lib()
    p = good_params(num_splits=8)
    fake = ctypes.c_void_p(1 << 20)
    i64 = ctypes.c_int64
    ok = (i64(32 * 4 * 128), i64(4 * 128), i64(128))
    assert lib.mlra_absorb_query(fake, fake, fake, ctypes.byref(p), 64, *ok, None) == -3      # d_nope
    assert lib.mlra_absorb_query(None, fake, fake, ctypes.byref(p), 128, *ok, None) == -1     # NULL q_pre
    assert lib.mlra_absorb_query(ctypes.c_void_p((1 << 20) + 8), fake, fake, ctypes.byref(p), 128, *ok,
                                 None) == -4                                                  # misaligned q_pre
    assert lib.mlra_absorb_query(fake, fake, fake, ctypes.byref(p), 128, i64(32 * 4 * 128), i64(4 * 128),
                                 i64(4), None) == -4                                          # 8-byte stride
    assert lib.mlra_absorb_query(fake, fake, fake, ctypes.byref(p), 128, i64(-1), *ok[1:], None) == -2


# ----------------------------------------------------------------- binding: host-side tensor checks
# Every mismatch below would send a kernel out of bounds if it reached the GPU. On this CPU-only
# run the binding must refuse each one with its own message, before the device check (which a
# fully consistent set of CPU tensors reaches last).

def _cpu_inputs(paged=False, **kw):
    from mlra_workloads import WORKLOADS, make_inputs
    w = WORKLOADS[5 if paged else 2].replace(B=3, h=8, lengths=("list", (40, 1, 70)), **kw)
    return w, make_inputs(w, seed=3)


def _decoder(inp, w, **over):
    import long_context_decode_mlra_amd as mlra
    args = dict(q_nope=inp.q_nope, q_rope=inp.q_rope, latent_cache=inp.latent, rope_cache=inp.rope,
                seqlens=inp.seqlens, W_UV=inp.W_UV, sm_scale=w.sm_scale, out_scale=w.gamma,
                max_seqlen=inp.max_seqlen, block_table=inp.block_table, page_size=w.page_size, num_splits=4)
    args.update(over)
    qn, qr, lat, rp = args.pop("q_nope"), args.pop("q_rope"), args.pop("latent_cache"), args.pop("rope_cache")
    return mlra.Decoder(qn, qr, lat, rp, **args)


@pytest.mark.parametrize("paged", [False, True])
def test_binding_consistent_cpu_tensors_reach_the_device_check(paged):
    w, inp = _cpu_inputs(paged)
    with pytest.raises(ValueError, match="must be GPU tensors"):
        _decoder(inp, w)


@pytest.mark.parametrize("case,match", [
    ("seqlens_short", "seqlens must be"), ("seqlens_int64", "seqlens must be"),
    ("q_rope_batch", "q_rope must be"), ("q_rope_heads", "q_rope must be"),
    ("latent_rows", "needs B \\* max_seqlen"), ("rope_rows", "one row numbering"),
    ("latent_heads", "latent_cache must be"), ("wuv_shape", "W_UV must be"), ("wuv_dtype", "W_UV must be"),
    ("wuv_strided", "W_UV must be"), ("out_shape", "out must be"), ("out_dtype", "out must be"),
    ("max_seqlen", "needs B \\* max_seqlen"), ("q_nope_3d", "q_nope must be"),
])
def test_binding_rejects_mismatched_tensors(case, match):
    import torch
    w, inp = _cpu_inputs()
    B, h = 3, 8
    over = {
        "seqlens_short": dict(seqlens=inp.seqlens[:2]),
        "seqlens_int64": dict(seqlens=inp.seqlens.long()),
        "q_rope_batch": dict(q_rope=inp.q_rope[:2]),
        "q_rope_heads": dict(q_rope=inp.q_rope[:, :4]),
        "latent_rows": dict(latent_cache=inp.latent[:-1], rope_cache=inp.rope[:-1]),
        "rope_rows": dict(rope_cache=inp.rope[:-1]),
        "latent_heads": dict(latent_cache=inp.latent[:, :2]),
        "wuv_shape": dict(W_UV=inp.W_UV[:, :4]),
        "wuv_dtype": dict(W_UV=inp.W_UV.to(torch.bfloat16)),
        "wuv_strided": dict(W_UV=inp.W_UV.transpose(2, 3)),
        "out_shape": dict(out=torch.empty(B, h, 64)),
        "out_dtype": dict(out=torch.empty(B, h, 128, dtype=torch.float64)),
        "max_seqlen": dict(max_seqlen=inp.max_seqlen + 1),
        "q_nope_3d": dict(q_nope=inp.q_nope.flatten(2)),
    }[case]
    with pytest.raises(ValueError, match=match):
        _decoder(inp, w, **over)


@pytest.mark.parametrize("case,match", [
    ("no_table", "block_table must be"), ("table_rows", "block_table must be"),
    ("table_cols", "fewer than max_seqlen"), ("table_int64", "block_table must be"),
    ("pool_empty", "less than one page"),
])
def test_binding_rejects_mismatched_paged_tensors(case, match):
    w, inp = _cpu_inputs(paged=True)
    bt = inp.block_table
    over = {
        "no_table": dict(block_table=None),
        "table_rows": dict(block_table=bt[:2]),
        "table_cols": dict(block_table=bt[:, :1].contiguous(), max_seqlen=max(inp.max_seqlen, 2 * w.page_size)),
        "table_int64": dict(block_table=bt.long()),
        "pool_empty": dict(latent_cache=inp.latent[:1], rope_cache=inp.rope[:1]),
    }[case]
    with pytest.raises(ValueError, match=match):
        _decoder(inp, w, **over)


def test_binding_rejects_table_for_contiguous_cache():
    w, inp = _cpu_inputs()
    import torch
    with pytest.raises(ValueError, match="page_size is 0"):
        _decoder(inp, w, block_table=torch.zeros(3, 2, dtype=torch.int32))


def test_gqa_binding_rejects_mismatched_tensors():
    import torch
    import long_context_decode_mlra_amd as mlra
    from mlra_workloads import GQA_WORKLOADS, make_gqa_inputs
    g = GQA_WORKLOADS["gqa_bf16_b32_hq64_hkv8_L32k"].replace(B=2, Hq=16, Hkv=2, lengths=("list", (33, 70)))
    gi = make_gqa_inputs(g, seed=1)
    kw = dict(sm_scale=g.sm_scale, max_seqlen=gi.max_seqlen, num_splits=4)
    with pytest.raises(ValueError, match="must be GPU tensors"):
        mlra.GqaDecoder(gi.q, gi.k_cache, gi.v_cache, seqlens=gi.seqlens, **kw)
    with pytest.raises(ValueError, match="seqlens must be"):
        mlra.GqaDecoder(gi.q, gi.k_cache, gi.v_cache, seqlens=gi.seqlens[:1], **kw)
    with pytest.raises(ValueError, match="needs B \\* max_seqlen"):
        mlra.GqaDecoder(gi.q, gi.k_cache[:-1], gi.v_cache[:-1], seqlens=gi.seqlens, **kw)
    with pytest.raises(ValueError, match="one row numbering"):
        mlra.GqaDecoder(gi.q, gi.k_cache, gi.v_cache[:-1], seqlens=gi.seqlens, **kw)
    with pytest.raises(ValueError, match="128 channels"):
        mlra.GqaDecoder(gi.q, gi.k_cache[..., :64], gi.v_cache[..., :64], seqlens=gi.seqlens, **kw)


def test_absorber_rejects_mismatched_tensors():
    import torch
    import long_context_decode_mlra_amd as mlra
    q_pre = torch.zeros(2, 8, 4, 128, dtype=torch.bfloat16)
    W_UK = torch.zeros(4, 8, 128, 128)
    q_nope = torch.zeros(2, 8, 4, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="must be GPU tensors"):
        mlra.Absorber(q_pre, W_UK, q_nope)
    with pytest.raises(ValueError, match="W_UK must be"):
        mlra.Absorber(q_pre, W_UK[:, :4], q_nope)
    with pytest.raises(ValueError, match="share one dtype"):
        mlra.Absorber(q_pre.float(), W_UK, q_nope)
    with pytest.raises(ValueError, match="q_pre must be"):
        mlra.Absorber(q_pre[:1], W_UK, q_nope)


def test_noalloc_refuses_oversized_workspace_before_any_device_call():
    """mlra_decode_noalloc checks the workspace its call needs against the fixed array first: with an
    explicit split count that check needs no device, so it runs here."""
    L = _lib()
    lib = L.lib()
    fake = ctypes.c_void_p(1 << 20)
    p = good_params(num_splits=8, batch=20000, num_heads=64)
    n = ctypes.c_size_t(0)
    assert lib.mlra_decode_workspace_size(ctypes.byref(p), ctypes.byref(n)) == 0
    assert n.value > L.MLRA_NOALLOC_SCRATCH_BYTES
    r = lib.mlra_decode_noalloc(fake, fake, fake, fake, None, fake, fake, fake, ctypes.byref(p), None)
    assert r == -5
    assert "mlra_decode_noalloc holds" in lib.mlra_last_error().decode()
    assert lib.mlra_decode_noalloc(fake, fake, fake, fake, None, fake, fake, fake, None, None) == -1
