"""HIP GQA decode comparator vs the fp64 GQA oracle, through the C ABI (needs an MI355X).

Tolerance as for the MLRA path (bf16 caches and queries, fp32 accumulation): max-abs
error <= 2e-2 and relative L2 error <= 5e-3 against the oracle on the same bf16 inputs.
"""
import numpy as np
import pytest
import torch

import oracle
from mlra_workloads import GQA_WORKLOADS, GqaInputs, make_gqa_inputs

pytestmark = pytest.mark.gpu

MAX_ABS, REL_L2 = 2e-2, 5e-3
W64 = GQA_WORKLOADS["gqa_bf16_b32_hq64_hkv8_L32k"]


def _mlra():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_decode_mlra_amd as mlra
    mlra.lib()  # raises if the library is missing: never a silent fallback
    return mlra


def gpu_gqa(inp, num_splits=0):
    mlra = _mlra()
    d = inp.to("cuda")
    out = mlra.gqa_decode(d.q, d.k_cache, d.v_cache, d.seqlens, sm_scale=inp.w.sm_scale,
                          max_seqlen=inp.max_seqlen, block_table=d.block_table, page_size=inp.w.page_size,
                          num_splits=num_splits)
    torch.cuda.synchronize()
    return out.cpu().double().numpy()


def assert_parity(got, ref, label=""):
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    diff = got - ref
    ma = float(np.abs(diff).max())
    rl = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-30))
    print(f"{label}: max_abs={ma:.3e} rel_l2={rl:.3e}", flush=True)
    assert ma <= MAX_ABS and rl <= REL_L2, f"{label}: max_abs={ma:.3e} rel_l2={rl:.3e}"


HEADS = {"hq64_hkv8": (64, 8), "hq32_hkv8": (32, 8), "mqa_hq16_hkv1": (16, 1), "mha_hq8_hkv8": (8, 8),
         "hq48_hkv3": (48, 3)}


@pytest.mark.parametrize("heads", sorted(HEADS))
@pytest.mark.parametrize("num_splits", [1, 3, 0])
def test_gqa_small_ragged(heads, num_splits):
    Hq, Hkv = HEADS[heads]
    w = W64.replace(B=4, Hq=Hq, Hkv=Hkv, lengths=("list", (1, 70, 333, 32)))
    inp = make_gqa_inputs(w, seed=21, poison=True, max_seqlen=352)
    assert_parity(gpu_gqa(inp, num_splits), oracle.gqa_decode_inputs(inp), label=f"{heads}/splits={num_splits}")


EDGE_LENGTHS = (0, 1, 2, 31, 32, 33, 63, 64, 65, 95, 96, 97, 0, 128, 129, 5)


@pytest.mark.parametrize("page_size", [0, 32, 64])
def test_gqa_edge_lengths_paged_and_poisoned(page_size):
    w = W64.replace(B=len(EDGE_LENGTHS), lengths=("list", EDGE_LENGTHS), page_size=page_size)
    inp = make_gqa_inputs(w, seed=22, poison=True, max_seqlen=192)
    ref = oracle.gqa_decode_inputs(inp)
    for splits in (0, 5, 64):
        got = gpu_gqa(inp, splits)
        assert np.all(got[[i for i, L in enumerate(EDGE_LENGTHS) if L == 0]] == 0)
        assert_parity(got, ref, label=f"page={page_size}/splits={splits}")


def test_gqa_large_logits_stay_finite():
    """Queries scaled by 40: logits in the hundreds; the online softmax must not overflow."""
    w = W64.replace(B=2, lengths=("list", (300, 77)))
    inp = make_gqa_inputs(w, seed=23)
    inp.q = (inp.q.float() * 40).to(torch.bfloat16)
    assert_parity(gpu_gqa(inp), oracle.gqa_decode_inputs(inp), label="large logits")


def test_gqa_deterministic_bitwise():
    w = W64.replace(B=3, lengths=("list", (1000, 2000, 17)))
    inp = make_gqa_inputs(w, seed=24)
    a, b = gpu_gqa(inp), gpu_gqa(inp)
    assert np.array_equal(a, b)


def test_gqa_full_size_sampled():
    """B=32, 64 query heads over 8 KV heads, L=32768 each (4 GiB of cache), in the launch
    configuration the benchmark times; the oracle checks sampled sequences."""
    mlra = _mlra()
    inp = make_gqa_inputs(W64, seed=1, device="cuda")
    print(f"GQA full size: B={W64.B} tokens={inp.total_tokens}", flush=True)
    sl = inp.seqlens.to("cuda")
    out = mlra.gqa_decode(inp.q, inp.k_cache, inp.v_cache, sl, sm_scale=W64.sm_scale, max_seqlen=inp.max_seqlen)
    torch.cuda.synchronize()
    got = out.cpu().double().numpy()
    assert np.all(np.isfinite(got))
    sel = (0, 19, 31)
    host = GqaInputs(
        w=W64, seqlens=inp.seqlens, max_seqlen=inp.max_seqlen, q=inp.q.cpu(), k_cache=inp.k_cache.cpu(),
        v_cache=inp.v_cache.cpu())
    ref = oracle.gqa_decode_inputs(host, batch_indices=sel)
    assert_parity(got[list(sel)], ref[list(sel)], label=f"GQA full size sampled {sel}")
