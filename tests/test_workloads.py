"""Seeded synthetic inputs: determinism, shapes, length draws and page-table structure; the
benchmark's one-GPU guard (CPU only)."""
import math
import os

import torch

from mlra_workloads import WORKLOADS, make_inputs


def test_same_seed_same_bytes():
    w = WORKLOADS[5].replace(B=6, lengths=("loguniform", 10, 300))
    a, b = make_inputs(w, seed=5), make_inputs(w, seed=5)
    def raw(t):
        return t.contiguous().view(-1).view(torch.uint8) if t.dtype.is_floating_point else t
    for k in ("seqlens", "q_nope", "q_rope", "latent", "rope", "W_UV", "block_table"):
        assert torch.equal(raw(getattr(a, k)), raw(getattr(b, k))), k
    c = make_inputs(w, seed=6)
    assert not torch.equal(a.latent, c.latent)


def test_length_draws_in_range():
    from mlra_workloads import draw_lengths
    gen = torch.Generator().manual_seed(3)
    Ls = draw_lengths(WORKLOADS[3], gen)
    assert len(Ls) == 4 and all(65536 <= L <= 131072 for L in Ls)
    gen = torch.Generator().manual_seed(5)
    Ls = draw_lengths(WORKLOADS[5], gen)
    assert len(Ls) == 64 and all(1024 <= L <= 65536 for L in Ls)
    # log-uniform: the median sits near the geometric mean sqrt(1024 * 65536) = 8192
    med = sorted(Ls)[32]
    assert 2048 < med < 32768


def test_page_table_is_a_permutation_of_the_pool():
    w = WORKLOADS[5].replace(B=7, lengths=("list", (1, 64, 65, 0, 200, 128, 3)))
    inp = make_inputs(w, seed=5)
    P = w.page_size
    used = []
    for b, L in enumerate(inp.seqlens.tolist()):
        n = (L + P - 1) // P
        row = inp.block_table[b].tolist()
        assert all(x >= 0 for x in row[:n]) and all(x == -1 for x in row[n:])
        used += row[:n]
    assert sorted(used) == list(range(len(used)))
    assert inp.latent.shape[0] == len(used) * P


def test_shapes_and_dtypes():
    for k, w in WORKLOADS.items():
        w = w.replace(B=2, lengths=("list", (33, 5)))
        inp = make_inputs(w, seed=k)
        B, h, NB, DL = 2, w.h, w.NB, w.DL
        assert inp.q_nope.shape == (B, h, NB, DL) and inp.q_rope.shape == (B, h, 64)
        assert inp.latent.shape[1:] == (NB, DL) and inp.rope.shape[1] == 64
        assert inp.W_UV.shape == (NB, h, DL, 128) and inp.W_UV.dtype == torch.float32
        assert inp.latent.dtype == w.torch_dtype
        if w.joint:
            row = NB * DL + 64  # 576, or 192 for one latent head
            assert inp.cache_joint.shape[1] == row and inp.q_joint.shape[-1] == row
            assert inp.latent.data_ptr() == inp.cache_joint.data_ptr()
            assert inp.rope.data_ptr() == inp.cache_joint.data_ptr() + NB * DL * inp.cache_joint.element_size()


def test_value_distributions():
    w = WORKLOADS[2].replace(B=2, lengths=("fixed", 4096))
    inp = make_inputs(w, seed=2)
    assert abs(inp.latent.float().std().item() - 1.0) < 0.02
    assert abs(inp.rope.float().std().item() - math.sqrt(3.0)) < 0.05
    assert abs(inp.W_UV.std().item() - 1.0 / math.sqrt(128)) < 0.002


def test_bench_refuses_more_than_one_gpu():
    """The benchmark runs on one GPU; asking for more exits with status 2 and says why, before any
    GPU work (no torch.distributed rendezvous, no device query)."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU only" in r.stderr and r.stdout == ""
