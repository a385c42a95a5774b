"""The fp64 oracle against facts that do not come from the oracle itself (CPU only)."""
import math

import numpy as np
import pytest

import oracle
import oracle_pins
from mlra_workloads import WORKLOADS, make_inputs


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.decode)


@pytest.mark.parametrize("chunk", [1, 2, 3, 7, 32, 1000])
def test_split_kv_equals_single_pass(chunk):
    """Split-KV partials merged with log-sum-exp weights equal the single pass (exact reformulation)."""
    rng = np.random.default_rng(30 + chunk)
    c = oracle_pins.tiny_case(rng, B=3, h=3, NB=4, DL=5, DR=2, DV=3, Ls=(37, 1, 64), scale=1.5)
    kw = dict(sm_scale=0.6, out_scale=0.5, max_seqlen=c["max_seqlen"])
    a = oracle.decode(c["q_nope"], c["q_rope"], c["latent"], c["rope"], c["W_UV"], c["seqlens"], **kw)
    s = oracle.decode_split(c["q_nope"], c["q_rope"], c["latent"], c["rope"], c["W_UV"], c["seqlens"],
                            chunk=chunk, **kw)
    np.testing.assert_allclose(s, a, rtol=1e-13, atol=1e-14)


def test_split_kv_real_widths_bf16_inputs():
    w = WORKLOADS[2].replace(B=2, lengths=("list", (300, 65)))
    inp = make_inputs(w, seed=2)
    a = oracle.decode_inputs(inp)
    s = oracle.decode_split(inp.q_nope, inp.q_rope, inp.latent, inp.rope, inp.W_UV, inp.seqlens,
                            sm_scale=w.sm_scale, out_scale=w.gamma, chunk=32, max_seqlen=inp.max_seqlen)
    np.testing.assert_allclose(s, a, rtol=1e-12, atol=1e-13)


def test_poisoned_rows_are_never_read():
    """NaN in every row no sequence owns (padding, unused page tails) must not reach the output."""
    for k in (3, 5):
        w = WORKLOADS[k].replace(B=3, lengths=("list", (70, 1, 129)))
        inp = make_inputs(w, seed=k, poison=True, max_seqlen=160)
        out = oracle.decode_inputs(inp)
        assert np.all(np.isfinite(out))


def test_per_token_bytes():
    """Both cache layouts hold 576 elements per token: 4 x 128 + 64 (MLRA-4) and 512 + 64 (MLA),
    i.e. 4.5 d_h with d_h = 128; one MLRA branch's logit space is 128 + 64 = 1.5 d_h."""
    for k in (1, 2, 3, 4, 5):
        assert WORKLOADS[k].token_elems == 576 == 4.5 * 128
    assert WORKLOADS[2].DL + WORKLOADS[2].DR == 192 == 1.5 * 128
    assert math.isclose(WORKLOADS[2].gamma, 0.5) and math.isclose(WORKLOADS[4].gamma, 1.0)
