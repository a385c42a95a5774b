"""mlra_decode_noalloc (the whole decode with the library's fixed per-device workspace) through
the C ABI against mlra_decode with a caller workspace: two calls in a row, the second on a
smaller batch, each identical to mlra_decode's output bit for bit and within the oracle
tolerance; a call whose workspace would exceed the fixed array is refused."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from mlra_workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

MAX_ABS, REL_L2 = 2e-2, 5e-3


def _mlra():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_decode_mlra_amd as mlra
    mlra.lib()
    return mlra


def _noalloc(mlra, dec):
    """One mlra_decode_noalloc call with the Decoder's tensors and parameters, into a fresh output."""
    from long_context_decode_mlra_amd._lib import check, lib
    qn, qr, lat, rp, bt, sl, W = dec.tensors
    out = torch.full_like(dec.out, float("nan"))
    ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    check(lib().mlra_decode_noalloc(ptr(qn), ptr(qr), ptr(lat), ptr(rp), ptr(bt), ptr(sl), ptr(W), ptr(out),
                                    ctypes.byref(dec.p), stream))
    return out


def _case(mlra, w, seed):
    inp = make_inputs(w, seed=seed, poison=True)
    d = inp.to("cuda")
    dec = mlra.Decoder(d.q_nope, d.q_rope, d.latent, d.rope, seqlens=d.seqlens, W_UV=d.W_UV, sm_scale=w.sm_scale,
                       out_scale=w.gamma, max_seqlen=inp.max_seqlen, block_table=d.block_table,
                       page_size=w.page_size)
    return inp, d, dec


def test_noalloc_matches_decode_twice_second_smaller():
    mlra = _mlra()
    cases = [WORKLOADS[5].replace(B=40, lengths=("list", tuple(range(1, 4001, 100)))),
             WORKLOADS[2].replace(B=3, lengths=("list", (700, 1, 64)))]
    for k, w in enumerate(cases):
        inp, d, dec = _case(mlra, w, seed=60 + k)
        print(f"noalloc case {k}: {w.name} B={w.B} workspace={dec.ws_bytes}", flush=True)
        assert dec.ws_bytes <= mlra.MLRA_NOALLOC_SCRATCH_BYTES
        got = _noalloc(mlra, dec)
        ref = dec().clone()
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"case {k}: mlra_decode_noalloc differs from mlra_decode"
        g = got.cpu().double().numpy()
        o = oracle.decode_inputs(inp)
        diff = g - o
        ma, rl = float(np.abs(diff).max()), float(np.linalg.norm(diff) / np.linalg.norm(o))
        print(f"  max_abs={ma:.3e} rel_l2={rl:.3e}", flush=True)
        assert ma <= MAX_ABS and rl <= REL_L2


def test_noalloc_refuses_a_workspace_past_its_array():
    mlra = _mlra()
    from long_context_decode_mlra_amd._lib import MlraError
    w = WORKLOADS[2].replace(B=2000, h=64, lengths=("list", (64,) * 2000))
    B, h = 2000, 64
    dev = "cuda"
    q_nope = torch.zeros(B, h, 4, 128, dtype=torch.bfloat16, device=dev)
    q_rope = torch.zeros(B, h, 64, dtype=torch.bfloat16, device=dev)
    lat = torch.zeros(B * 64, 4, 128, dtype=torch.bfloat16, device=dev)
    rope = torch.zeros(B * 64, 64, dtype=torch.bfloat16, device=dev)
    sl = torch.full((B,), 64, dtype=torch.int32, device=dev)
    W = torch.zeros(4, h, 128, 128, device=dev)
    dec = mlra.Decoder(q_nope, q_rope, lat, rope, seqlens=sl, W_UV=W, sm_scale=w.sm_scale, out_scale=0.5,
                       max_seqlen=64)
    assert dec.ws_bytes > mlra.MLRA_NOALLOC_SCRATCH_BYTES
    with pytest.raises(MlraError, match="MLRA_ERR_WORKSPACE"):
        _noalloc(mlra, dec)
