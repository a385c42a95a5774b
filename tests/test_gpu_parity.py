"""HIP decode path vs the fp64 oracle, element by element, through the C ABI (needs an MI355X).

Tolerance (bf16 caches and queries, fp32 accumulation): max-abs error <= 2e-2 and
relative L2 error <= 5e-3 against the fp64 oracle on the same bf16 inputs. The fp32
path is held to rel-L2 <= 1e-4 as well (fp32 inputs, fp32 MFMA and softmax).
"""
import math

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
    mlra.lib()  # raises if the library is missing: never a silent fallback
    return mlra


def gpu_decode(inp, num_splits=0):
    mlra = _mlra()
    d = inp.to("cuda")
    w = inp.w
    out = mlra.decode(d.q_nope, d.q_rope, d.latent, d.rope, d.seqlens, d.W_UV, sm_scale=w.sm_scale,
                      out_scale=w.gamma, max_seqlen=inp.max_seqlen, block_table=d.block_table,
                      page_size=w.page_size, num_splits=num_splits)
    torch.cuda.synchronize()
    return out.cpu().double().numpy()


def errors(got, ref):
    diff = got - ref
    return float(np.abs(diff).max()), float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-30))


def assert_parity(got, ref, max_abs=MAX_ABS, rel_l2=REL_L2, label=""):
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    ma, rl = errors(got, ref)
    print(f"{label}: max_abs={ma:.3e} rel_l2={rl:.3e}", flush=True)
    assert ma <= max_abs and rl <= rel_l2, f"{label}: max_abs={ma:.3e} rel_l2={rl:.3e}"


SMALL = {
    "mlra4_bf16": WORKLOADS[2],
    "mla_bf16": WORKLOADS[4],
    # MLA at the scale of its own 576-channel logit (the workloads use 1/sqrt(192) for both forms)
    "mla_bf16_scale576": WORKLOADS[4].replace(sm_scale=1.0 / math.sqrt(576.0)),
    "mlra2_bf16": WORKLOADS[2].replace(name="mlra2", NB=2, DL=256, rope_std=1.0),
    "mlra4_f32": WORKLOADS[1].replace(h=32),
    "mla_f32": WORKLOADS[4].replace(dtype="f32"),
}


@pytest.mark.parametrize("name", sorted(SMALL))
@pytest.mark.parametrize("num_splits", [1, 3, 0])
def test_small_ragged(name, num_splits):
    w = SMALL[name].replace(B=3, lengths=("list", (1, 70, 333)))
    inp = make_inputs(w, seed=7, poison=True, max_seqlen=352)
    got = gpu_decode(inp, num_splits)
    ref = oracle.decode_inputs(inp)
    tol = dict(rel_l2=1e-4, max_abs=1e-3) if w.dtype == "f32" else {}
    assert_parity(got, ref, label=f"{name}/splits={num_splits}", **tol)


@pytest.mark.parametrize("name", ["mla_bf16", "mlra2_bf16", "mlra4_f32", "mla_f32"])
@pytest.mark.parametrize("page_size", [32, 64])
def test_paged_every_form(name, page_size):
    """Paged caches (random page permutation, NaN in unowned rows) for the forms beyond MLRA-4
    bf16: the split-head kernel (MLA joint rows, MLRA-2) and the fp32 kernels."""
    w = SMALL[name].replace(B=4, lengths=("list", (1, 70, 333, 64)), page_size=page_size)
    inp = make_inputs(w, seed=9, poison=True)
    tol = dict(rel_l2=1e-4, max_abs=1e-3) if w.dtype == "f32" else {}
    for splits in (0, 7):
        assert_parity(gpu_decode(inp, splits), oracle.decode_inputs(inp), label=f"{name}/page={page_size}/splits={splits}", **tol)


@pytest.mark.parametrize("cfg", [2, 5, 1])
def test_mlra4_joint_rows(cfg):
    """MLRA-4 with queries and cache stored as joint rows ([.., 576]: the four latent heads, then
    RoPE), so every query and cache stride differs from the separate-tensor layout: contiguous and
    paged bf16 (one wave per branch) and fp32 (whole tiles)."""
    w = WORKLOADS[cfg].replace(B=4, lengths=("list", (1, 70, 333, 64)), joint=True)
    inp = make_inputs(w, seed=13, poison=True)
    tol = dict(rel_l2=1e-4, max_abs=1e-3) if w.dtype == "f32" else {}
    ref = oracle.decode_inputs(inp)
    for splits in (0, 5):
        assert_parity(gpu_decode(inp, splits), ref, label=f"joint cfg{cfg}/splits={splits}", **tol)


EDGE_LENGTHS = (0, 1, 2, 31, 32, 33, 63, 64, 65, 95, 96, 97, 0, 128, 129, 5)


@pytest.mark.parametrize("paged", [False, True])
def test_edge_lengths_and_poisoned_padding(paged):
    w = WORKLOADS[5 if paged else 3].replace(B=len(EDGE_LENGTHS), lengths=("list", EDGE_LENGTHS))
    inp = make_inputs(w, seed=11, poison=True, max_seqlen=192)
    for splits in (0, 5, 64):
        got = gpu_decode(inp, splits)
        ref = oracle.decode_inputs(inp)
        assert_parity(got, ref, label=f"edge paged={paged} splits={splits}")
        for b, L in enumerate(EDGE_LENGTHS):
            if L == 0:
                assert np.all(got[b] == 0.0)


@pytest.mark.parametrize("h", [1, 5, 8, 16, 33, 48, 64])
def test_head_counts(h):
    """Head counts below, between and at the 32-head blocks (1 and 5 leave most MFMA columns
    empty; 33 puts one head in a second block)."""
    w = WORKLOADS[2].replace(B=2, h=h, lengths=("list", (200, 45)))
    inp = make_inputs(w, seed=h)
    assert_parity(gpu_decode(inp), oracle.decode_inputs(inp), label=f"h={h}")
    wm = WORKLOADS[4].replace(B=2, h=h, lengths=("list", (90, 260)))
    inp = make_inputs(wm, seed=h + 1)
    assert_parity(gpu_decode(inp), oracle.decode_inputs(inp), label=f"mla h={h}")


def test_cfg1_full_f32():
    """fp32 everywhere, B=1, h=16, L=1024 (the whole workload)."""
    inp = make_inputs(WORKLOADS[1], seed=1)
    got = gpu_decode(inp)
    ref = oracle.decode_inputs(inp)
    assert_parity(got, ref, label="cfg1", rel_l2=1e-4, max_abs=1e-3)


def test_large_logits_stay_finite():
    """Logits of several hundred: the online softmax must not overflow."""
    w = WORKLOADS[2].replace(B=2, lengths=("list", (300, 64)), sm_scale=1.0)
    inp = make_inputs(w, seed=3)
    inp.q_rope.mul_(4)
    got = gpu_decode(inp)
    ref = oracle.decode_inputs(inp)
    # Near-one-hot attention: compare relative to the output scale.
    assert_parity(got, ref, max_abs=2e-2 * float(np.abs(ref).max()), label="large logits")


def test_deterministic_bitwise():
    w = WORKLOADS[5].replace(B=5, lengths=("list", (1000, 64, 3000, 1, 777)))
    inp = make_inputs(w, seed=5)
    a = gpu_decode(inp)
    b = gpu_decode(inp)
    assert np.array_equal(a, b)


def test_split_counts_agree():
    w = WORKLOADS[2].replace(B=4, lengths=("list", (2000, 31, 4096, 700)))
    inp = make_inputs(w, seed=9)
    ref = oracle.decode_inputs(inp)
    outs = []
    for splits in (1, 2, 7, 33, 250, 0):
        got = gpu_decode(inp, splits)
        assert_parity(got, ref, label=f"splits={splits}")
        outs.append(got)
    # Each split rounds its attention weights to bf16 relative to its own running max, so
    # different split counts differ by about the weight rounding (2^-9 per weight, averaged):
    # the same order as the error against the oracle, far inside the gate.
    for o in outs[1:]:
        assert errors(o, outs[0])[1] < 2e-3


def test_plan_partitions_tiles():
    """Split planning (integer, exact): split g holds exactly the global tiles [g*T/G, (g+1)*T/G);
    every tile of every sequence exactly once, in order."""
    mlra = _mlra()
    rng = np.random.default_rng(0)
    for trial in range(12):
        B = int(rng.integers(1, 70))
        Ls = rng.integers(0, 5000, size=B)
        Ls[rng.random(B) < 0.2] = 0
        G_req = int(rng.integers(1, 600))
        seqlens = torch.tensor(Ls, dtype=torch.int32, device="cuda")
        segs, T, G = mlra.plan(seqlens, G_req, max_segments=B + 1)
        tiles = [(int(L) + 31) // 32 for L in Ls]
        first = np.concatenate([[0], np.cumsum(tiles)])  # first global tile of each sequence
        assert T == sum(tiles) and G == min(G_req, T)
        seen = []
        for g in range(G_req):
            flat = []
            for (b, ta, te) in segs[g].tolist():
                if b < 0:
                    continue
                assert g < G and 0 <= ta < te <= tiles[b]
                seen += [(b, t) for t in range(ta, te)]
                flat += [int(first[b]) + t for t in range(ta, te)]
            if g < G:  # exactly the global tiles [g*T/G, (g+1)*T/G)
                assert flat == list(range(g * T // G, (g + 1) * T // G))
        assert seen == [(b, t) for b in range(B) for t in range(tiles[b])]


def test_copy_and_read_probes():
    mlra = _mlra()
    src = torch.randn(1 << 20, device="cuda")
    dst = torch.empty_like(src)
    mlra.copy_bandwidth_probe(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    words = torch.randint(-2**31, 2**31 - 1, (1 << 20,), dtype=torch.int32)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    mlra.read_bandwidth_probe(words.cuda(), sink)
    expect = 0
    for v in words.numpy().view(np.uint32).reshape(-1, 4).T:
        expect ^= int(np.bitwise_xor.reduce(v))
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == expect


# ----------------------------------------------------------------- the one-latent-head shard form
SHARD = WORKLOADS[7]


@pytest.mark.parametrize("page_size", [0, 64])
@pytest.mark.parametrize("num_splits", [1, 3, 0])
def test_shard_small_ragged(page_size, num_splits):
    """One latent head of 128 channels in joint 192-wide rows (one GPU's share of MLRA-4), ragged
    lengths with NaN in every row no sequence owns; contiguous and paged."""
    w = SHARD.replace(B=3, lengths=("list", (1, 70, 333)), page_size=page_size)
    inp = make_inputs(w, seed=17, poison=True, max_seqlen=352)
    assert_parity(gpu_decode(inp, num_splits), oracle.decode_inputs(inp),
                  label=f"shard page={page_size}/splits={num_splits}")


def test_shard_edge_lengths():
    w = SHARD.replace(B=len(EDGE_LENGTHS), lengths=("list", EDGE_LENGTHS), joint=False)
    inp = make_inputs(w, seed=18, poison=True, max_seqlen=192)
    ref = oracle.decode_inputs(inp)
    for splits in (0, 5, 64):
        got = gpu_decode(inp, splits)
        assert_parity(got, ref, label=f"shard edge splits={splits}")
        for b, L in enumerate(EDGE_LENGTHS):
            if L == 0:
                assert np.all(got[b] == 0.0)


def test_shard_deterministic_bitwise():
    w = SHARD.replace(B=5, lengths=("list", (1000, 64, 3000, 1, 777)))
    inp = make_inputs(w, seed=20)
    assert np.array_equal(gpu_decode(inp), gpu_decode(inp))


def test_four_shards_sum_to_mlra4():
    """The four latent heads of an MLRA-4 cache decoded apart, each from views of the MLRA-4
    tensors with its own W_UV block, and summed: the MLRA-4 output (the branch sum done across
    GPUs in the tensor-parallel layout), against the oracle and against the MLRA-4 kernel."""
    mlra = _mlra()
    w = WORKLOADS[2].replace(B=4, lengths=("list", (1000, 64, 3000, 777)))
    inp = make_inputs(w, seed=19)
    d = inp.to("cuda")
    total = torch.zeros(4, w.h, 128, dtype=torch.float64, device="cuda")
    for j in range(4):
        out = mlra.decode(d.q_nope[:, :, j:j + 1], d.q_rope, d.latent[:, j:j + 1], d.rope, d.seqlens,
                          d.W_UV[j:j + 1], sm_scale=w.sm_scale, out_scale=w.gamma, max_seqlen=inp.max_seqlen)
        total += out.double()
    torch.cuda.synchronize()
    total = total.cpu().numpy()
    assert_parity(total, oracle.decode_inputs(inp), label="sum of 4 shards vs oracle")
    assert_parity(total, gpu_decode(inp), label="sum of 4 shards vs MLRA-4 kernel")


# ----------------------------------------------------------------- full-size workloads, sampled sequences
FULL = {2: tuple(range(32)), 3: (0, 1, 2, 3), 4: (0, 31), 5: (0, 13, 40, 63), 6: (0, 31), 7: (0, 31)}


@pytest.mark.parametrize("cfg", sorted(FULL))
def test_full_size_sampled(cfg):
    """The workload at its full size in the launch configuration the benchmark times
    (num_splits = one per resident slot); the oracle checks sampled sequences (every sequence
    of the B=32, L=32K MLRA-4 workload)."""
    w = WORKLOADS[cfg]
    inp = make_inputs(w, seed=cfg)
    print(f"cfg{cfg}: B={w.B} tokens={inp.total_tokens} max_seqlen={inp.max_seqlen}", flush=True)
    got = gpu_decode(inp, 0)
    sel = FULL[cfg]
    ref = oracle.decode_inputs(inp, batch_indices=sel)
    assert np.all(np.isfinite(got))
    assert_parity(got[list(sel)], ref, label=f"cfg{cfg} sampled {sel}")


def test_mla_full_size_scale_576():
    """Absorbed MLA at its full size with the softmax scale of a 576-channel logit, 1/sqrt(576)."""
    w = WORKLOADS[4].replace(sm_scale=1.0 / math.sqrt(576.0))
    inp = make_inputs(w, seed=4)
    got = gpu_decode(inp, 0)
    sel = (0, 9, 31)
    ref = oracle.decode_inputs(inp, batch_indices=sel)
    assert np.all(np.isfinite(got))
    assert_parity(got[list(sel)], ref, label=f"cfg4 scale 1/sqrt(576) sampled {sel}")


def test_two_sequence_groups_and_workspace_reuse():
    """B=40: one full group of 32 sequences and a partial one; the same Decoder (and workspace)
    is called three times in a row and must give the same bits."""
    mlra = _mlra()
    rng = np.random.default_rng(40)
    Ls = tuple(int(x) for x in rng.integers(0, 900, size=40))
    w = WORKLOADS[2].replace(B=40, lengths=("list", Ls))
    inp = make_inputs(w, seed=40, poison=True)
    d = inp.to("cuda")
    dec = mlra.Decoder(d.q_nope, d.q_rope, d.latent, d.rope, seqlens=d.seqlens, W_UV=d.W_UV, sm_scale=w.sm_scale,
                       out_scale=w.gamma, max_seqlen=inp.max_seqlen)
    outs = []
    for _ in range(3):
        outs.append(dec().cpu().double().numpy())
        torch.cuda.synchronize()
    ref = oracle.decode_inputs(inp)
    assert_parity(outs[0], ref, label="B=40")
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


@pytest.mark.parametrize("cfg,B,h", [(7, 40, 32), (2, 45, 4)])
def test_combine_runs_across_groups(cfg, B, h):
    """Batches past one 32-sequence group whose combine grid alone would not fill the device, so a
    combine workgroup takes a shorter run of sequences: runs of 8 for the shard form at B=40, h=32,
    of 4 for MLRA-4 at B=45, h=4 (the last run holds one sequence)."""
    rng = np.random.default_rng(43 + B)
    Ls = tuple(int(x) for x in rng.integers(0, 700, size=B))
    w = WORKLOADS[cfg].replace(B=B, h=h, lengths=("list", Ls))
    inp = make_inputs(w, seed=43, poison=True)
    print(f"{w.name} B={B} h={h}", flush=True)
    got = gpu_decode(inp, 0)
    assert_parity(got, oracle.decode_inputs(inp), label=f"{w.name} B={B} h={h}")


def test_one_sequence_of_a_million_tokens():
    """Maximum length on one GPU-resident sequence: B=1, L=2^20 (1.2 GB of cache). Every split
    of the default launch falls in the same sequence, so the combine merges 512+1 slots for it."""
    w = WORKLOADS[2].replace(B=1, lengths=("list", (1 << 20,)))
    inp = make_inputs(w, seed=41)
    print(f"B=1 L={1 << 20}", flush=True)
    got = gpu_decode(inp, 0)
    assert_parity(got, oracle.decode_inputs(inp), label="B=1 L=2^20")


def test_a_thousand_short_sequences():
    """B=1000 ragged sequences of 0..100 tokens (32 sequence groups in the combine; splits of
    one or two tiles that span several sequences), paged and contiguous; and the shard form, paged."""
    rng = np.random.default_rng(42)
    Ls = tuple(int(x) for x in rng.integers(0, 101, size=1000))
    for w in (WORKLOADS[2].replace(B=1000, lengths=("list", Ls)), WORKLOADS[5].replace(B=1000, lengths=("list", Ls)),
              WORKLOADS[7].replace(B=1000, lengths=("list", Ls), page_size=64)):
        inp = make_inputs(w, seed=42, poison=True)
        got = gpu_decode(inp, 0)
        assert np.all(got[[b for b, L in enumerate(Ls) if L == 0]] == 0)
        assert_parity(got, oracle.decode_inputs(inp), label=f"B=1000 {w.name} page={w.page_size}")


@pytest.mark.parametrize("cfg", [5, 7, 4])
def test_graph_replay_matches_eager(cfg):
    """A captured decode step replayed several times, with eager work in between, gives the
    eager result every time (the step records kernel launches only): paged MLRA-4, the shard form
    (whose combine runs over short sequence runs) and MLA."""
    mlra = _mlra()
    w = WORKLOADS[cfg].replace(B=6, lengths=("list", (700, 1, 2048, 65, 0, 333)))
    inp = make_inputs(w, seed=12)
    d = inp.to("cuda")
    dec = mlra.Decoder(d.q_nope, d.q_rope, d.latent, d.rope, seqlens=d.seqlens, W_UV=d.W_UV, sm_scale=w.sm_scale,
                       out_scale=w.gamma, max_seqlen=inp.max_seqlen, block_table=d.block_table,
                       page_size=w.page_size)
    eager = dec().clone()
    torch.cuda.synchronize()
    graph = dec.capture_graph()
    for k in range(4):
        dec.out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(dec.out, eager), f"replay {k}"
        junk = torch.randn(1 << 16, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
    assert_parity(eager.cpu().double().numpy(), oracle.decode_inputs(inp), label=f"graph cfg{cfg}")


@pytest.mark.parametrize("cfg", [2, 5])
def test_graph_of_several_steps(cfg):
    """Eight decode steps recorded in one graph: every replay leaves the eager result (each step
    clears the combine's arrival counters itself, so back-to-back steps in a graph stay exact)."""
    mlra = _mlra()
    w = WORKLOADS[cfg].replace(B=5, lengths=("list", (900, 33, 0, 2048, 64)))
    inp = make_inputs(w, seed=13)
    d = inp.to("cuda")
    dec = mlra.Decoder(d.q_nope, d.q_rope, d.latent, d.rope, seqlens=d.seqlens, W_UV=d.W_UV, sm_scale=w.sm_scale,
                       out_scale=w.gamma, max_seqlen=inp.max_seqlen, block_table=d.block_table,
                       page_size=w.page_size)
    eager = dec().clone()
    torch.cuda.synchronize()
    graph = dec.capture_graph(steps=8)
    for k in range(3):
        dec.out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(dec.out, eager), f"replay {k}"
        junk = torch.randn(1 << 16, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
    with pytest.raises(ValueError):
        dec.capture_graph(steps=0)
    assert_parity(eager.cpu().double().numpy(), oracle.decode_inputs(inp), label=f"graph x8 cfg{cfg}")


@pytest.mark.parametrize("cfg", [2, 7, 4])
def test_combine_reruns_on_the_same_partials(cfg):
    """The combine counts its workgroups per (query head, run of sequences) and the last one of a
    head adds the branch blocks: after one attention launch, three combine launches in a row each
    give the full decode's bits (the counters are back at zero after every combine)."""
    mlra = _mlra()
    w = WORKLOADS[cfg].replace(B=37, lengths=("list", tuple(range(1, 37 * 53, 53))))
    inp = make_inputs(w, seed=70 + cfg)
    d = inp.to("cuda")
    dec = mlra.Decoder(d.q_nope, d.q_rope, d.latent, d.rope, seqlens=d.seqlens, W_UV=d.W_UV, sm_scale=w.sm_scale,
                       out_scale=w.gamma, max_seqlen=inp.max_seqlen)
    full = dec().clone()
    dec.splitkv()
    for k in range(3):
        dec.out.fill_(float("nan"))
        dec.combine()
        torch.cuda.synchronize()
        assert torch.equal(dec.out, full), f"combine run {k}"
    assert_parity(full.cpu().double().numpy(), oracle.decode_inputs(inp), label=f"rerun cfg{cfg}")

def test_two_streams_two_workspaces():
    """Two decodes with their own workspaces, enqueued on two streams (default priority) so that
    they may run at the same time, give the bits each gives alone."""
    mlra = _mlra()
    decs, alone = [], []
    for k, w in enumerate((WORKLOADS[2].replace(B=3, lengths=("list", (2000, 31, 900))),
                           WORKLOADS[5].replace(B=4, lengths=("list", (700, 1, 1500, 64))))):
        inp = make_inputs(w, seed=50 + k)
        d = inp.to("cuda")
        dec = mlra.Decoder(d.q_nope, d.q_rope, d.latent, d.rope, seqlens=d.seqlens, W_UV=d.W_UV, sm_scale=w.sm_scale,
                           out_scale=w.gamma, max_seqlen=inp.max_seqlen, block_table=d.block_table,
                           page_size=w.page_size)
        alone.append(dec().clone())
        decs.append((dec, d))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        for (dec, _), st in zip(decs, streams):
            dec.out.fill_(float("nan"))
        torch.cuda.synchronize()
        for (dec, _), st in zip(decs, streams):
            with torch.cuda.stream(st):
                dec(st)
        torch.cuda.synchronize()
        for (dec, _), ref in zip(decs, alone):
            assert torch.equal(dec.out, ref), f"rep {rep}"


# ----------------------------------------------------------------- query-side absorption (decode step 1)
from mlra_workloads import make_absorption_inputs


@pytest.mark.parametrize("cfg,shared", [(2, False), (2, True), (4, False), (1, False), (7, False)])
def test_absorb_query_then_decode(cfg, shared):
    """GPU absorption q_nope = W_UK q_pre against the oracle's, then the full three-step decode
    (absorb on the GPU, attend, up-project) against the oracle on the fp64 absorbed query."""
    mlra = _mlra()
    w = WORKLOADS[cfg].replace(B=3, lengths=("list", (257, 1, 90)))
    inp = make_inputs(w, seed=cfg, max_seqlen=288)
    q_pre, W_UK = make_absorption_inputs(w, seed=cfg, B=3, shared_query=shared)
    d = inp.to("cuda")
    q_pre_d = q_pre.to("cuda") if not shared else q_pre[:, :, :1].to("cuda").expand_as(q_pre)
    q_nope = torch.empty(3, w.h, w.NB, w.DL, dtype=w.torch_dtype, device="cuda")
    mlra.absorb_query(q_pre_d, W_UK.to("cuda"), q_nope)
    torch.cuda.synchronize()
    ref_q = oracle.absorb(q_pre, W_UK)
    got_q = q_nope.cpu().double().numpy()
    # bf16 output: one rounding to nearest (relative 2^-9) of an fp32-accumulated dot product.
    bound = (2.0 ** -8 if w.dtype == "bf16" else 1e-5) * np.abs(ref_q) + 1e-5
    assert np.all(np.abs(got_q - ref_q) <= bound), float(np.max(np.abs(got_q - ref_q) - bound))
    out = mlra.decode(q_nope, d.q_rope, d.latent, d.rope, d.seqlens, d.W_UV, sm_scale=w.sm_scale,
                      out_scale=w.gamma, max_seqlen=inp.max_seqlen)
    torch.cuda.synchronize()
    ref = oracle.decode(ref_q, inp.q_rope, inp.latent, inp.rope, inp.W_UV, inp.seqlens, sm_scale=w.sm_scale,
                        out_scale=w.gamma, max_seqlen=inp.max_seqlen)
    tol = dict(rel_l2=1e-4, max_abs=1e-3) if w.dtype == "f32" else {}
    assert_parity(out.cpu().double().numpy(), ref, label=f"absorb+decode cfg{cfg} shared={shared}", **tol)
