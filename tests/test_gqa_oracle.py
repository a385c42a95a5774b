"""The fp64 GQA oracle against its pins, and one planted mistake at a time caught by them (CPU only)."""
import numpy as np
import pytest

import gqa_pins
import oracle
from oracle import gqa_oracle as G
from mlra_workloads import GQA_WORKLOADS, make_gqa_inputs


@pytest.mark.parametrize("pin", gqa_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.gqa_decode)


def _caught():
    failures = []
    for pin in gqa_pins.ALL_PINS:
        try:
            pin(G.gqa_decode)
        except Exception as e:  # any error counts as the mutant being caught
            failures.append((pin.__name__, type(e).__name__))
    return failures


def _group_modulo(i, Hq, Hkv):
    return i % Hkv


def _group_of_next(i, Hq, Hkv):
    return min(i // (Hq // Hkv) + 1, Hkv - 1) if Hkv > 1 else 0


def _kv_swapped(q_i, K, V, sm_scale):
    s = sm_scale * (V @ q_i)
    w = np.exp(s - s.max())
    return (w @ K) / w.sum()


def _scale_missing(q_i, K, V, sm_scale):
    s = K @ q_i
    w = np.exp(s - s.max())
    return (w @ V) / w.sum()


def _no_max(q_i, K, V, sm_scale):
    with np.errstate(over="ignore", invalid="ignore"):
        w = np.exp(sm_scale * (K @ q_i))
        return (w @ V) / w.sum()


def _unnormalised(q_i, K, V, sm_scale):
    s = sm_scale * (K @ q_i)
    return np.exp(s - s.max()) @ V


def _rows_ignore_table(b, L, block_table, page_size, max_seqlen):
    return b * int(max_seqlen) + np.arange(L, dtype=np.int64)


MUTANTS = {
    "group_modulo": ("gqa_group_of", _group_modulo),
    "group_off_by_one": ("gqa_group_of", _group_of_next),
    "kv_swapped": ("gqa_head_attention", _kv_swapped),
    "scale_missing": ("gqa_head_attention", _scale_missing),
    "no_max": ("gqa_head_attention", _no_max),
    "unnormalised": ("gqa_head_attention", _unnormalised),
    "rows_ignore_table": ("physical_rows", _rows_ignore_table),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(G, attr, fn)
    assert _caught(), f"mutant {name} passed every GQA pin"


def test_unmutated_oracle_passes_every_pin():
    assert _caught() == []


def test_generated_workload_shapes_and_oracle_run():
    w = GQA_WORKLOADS["gqa_bf16_b32_hq64_hkv8_L32k"].replace(B=2, lengths=("list", (33, 0)), page_size=32)
    inp = make_gqa_inputs(w, seed=3, poison=True)
    assert inp.q.shape == (2, 64, 128) and inp.k_cache.shape[1:] == (8, 128)
    out = oracle.gqa_decode_inputs(inp)
    assert np.all(np.isfinite(out)) and np.all(out[1] == 0)
