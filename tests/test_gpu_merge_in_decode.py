"""The balanced split's merge inside the decode kernel (the worker whose piece
is counted last combines a split sequence; the new tokens are stored by the
same launch): the workspace's arrival counters are left zero by every call,
whatever the shapes and split modes that share the workspace; a captured
graph of fused steps replays to the eager result bit for bit; and the
outputs match the oracle at the usual tolerance."""

import sys

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_131_amd import binding as pb
from paged_kv_cache_131_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL = 2e-3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def device_case(w):
    et = w.cfg.etype
    return {
        "q": pb.to_device(w.q, et, DEV),
        "kc": pb.to_device(w.k_cache, et, DEV),
        "vc": pb.to_device(w.v_cache, et, DEV),
        "kn": pb.to_device(w.k_new, et, DEV),
        "vn": pb.to_device(w.v_new, et, DEV),
        "bt": pb.int32_to_device(w.block_tables, DEV),
        "cl": pb.int32_to_device(w.context_lens, DEV),
    }


def fused_step(w, d, ws, part=pb.PA_PARTITION_AUTO, out=None):
    if out is None:
        out = torch.empty(d["q"].shape, dtype=torch.float32, device=DEV)
    pb.pa_write_decode(out, d["q"], d["kn"], d["vn"], d["kc"], d["vc"], d["bt"], d["cl"], w.cfg.scale,
                       w.max_context_len, partition_size=part, workspace=ws)
    return out


def oracle_out(w, seqs=None):
    kr, vr = oracle.write_kv(w.k_cache, w.v_cache, w.k_new, w.v_new, w.slot_mapping, w.cfg.block_size)
    return oracle.decode(w.q, kr, vr, w.block_tables, w.context_lens, w.cfg.scale, w.cfg.block_size, w.cfg.etype,
                         seqs=seqs)


def check(got, ref, label, seqs=None, tol=TOL):
    g = got.float().cpu().numpy().astype(np.float64)
    if seqs is not None:
        g, ref = g[seqs], ref[seqs]
    err = float(np.abs(g - ref).max())
    say(f"  {label}: max |gpu - oracle| = {err:.3e}")
    assert np.all(np.isfinite(g)) and err <= tol, label


def mixed_lengths(S, seed):
    """Mostly short contexts (1-4 chunks), every 101st one of 1,500-3,000
    tokens and one of 8,000: with this many sequences every worker holds a
    few, so sequences cut at worker boundaries have two pieces, the 8,000-token
    one about ten or more (more than one batch of the merge's loads)."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, 121, size=S)
    lens[::101] = rng.integers(1500, 3001, size=len(lens[::101]))
    lens[7] = 8000
    return lens.astype(np.int32)


@pytest.mark.parametrize("etype,d,Hq,Hkv,B,algo,fused", [
    ("bf16", 128, 32, 8, 16, "auto", True),     # Llama-3-8B heads, g = 4
    ("f16", 64, 16, 2, 32, "mfma", False),      # g = 8, head_dim 64
    ("bf16", 128, 40, 8, 16, "mfma", True),     # g = 5
    ("f32", 128, 16, 8, 16, "vector", True),    # the vector engine (fp32), g = 2
    ("bf16", 64, 8, 8, 64, "vector", False),    # the vector engine, g = 1, 64-token blocks
])
def test_in_kernel_merge_many_sequences(etype, d, Hq, Hkv, B, algo, fused):
    """1,024 sequences (at least a quarter as many as any launch has workers
    per KV head, so the decode kernel merges itself): every output against the
    oracle, for both engines, with and without the fused write, and the
    arrival counters left zero."""
    S = 1024
    lens = mixed_lengths(S, 70 + Hq)
    cfg = wl.DecodeConfig(f"mixed-{etype}-{Hq}-{Hkv}", 70 + Hq, S, Hq, Hkv, d, B, etype,
                          d ** -0.5, ("fixed", tuple(int(x) for x in lens)), int(lens.max()))
    say(f"in-kernel merge: {etype} d={d} Hq={Hq} Hkv={Hkv} B={B} {algo} fused={fused}")
    w = wl.make_decode_workload(cfg, lengths=lens)
    dv = device_case(w)
    need = pb.pa_decode_workspace_bytes(S, Hq, Hkv, d, w.max_context_len, -1)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    out = torch.empty(dv["q"].shape, dtype=torch.float32, device=DEV)
    if fused:
        fused_step(w, dv, ws, out=out)
        ref = oracle_out(w)
    else:
        pb.pa_write_kv(dv["kn"], dv["vn"], dv["kc"], dv["vc"], pb.int32_to_device(w.slot_mapping, DEV))
        pb.pa_decode(out, dv["q"], dv["kc"], dv["vc"], dv["bt"], dv["cl"], cfg.scale, w.max_context_len,
                     workspace=ws, algo=algo)
        ref = oracle_out(w)
    torch.cuda.synchronize()
    check(out, ref, "all sequences", tol=1e-5 if etype == "f32" else TOL)
    assert int(ws[:pb.WORKSPACE_COUNTER_BYTES].count_nonzero()) == 0


def test_counters_left_zero_across_shapes_and_modes():
    """One zero-filled workspace serves, in turn, balanced splits of two
    shapes (1 and 96 sequences, so different workers hold the first pieces),
    fixed 64-token partitions and the shared split; after each call the
    counter region is zero and the output matches the oracle."""
    cases = [
        (wl.DecodeConfig("one-long", 61, 1, 32, 8, 128, 16, "bf16", 0.088, ("fixed", (9000,)), 9000), -1),
        (wl.DecodeConfig("ragged-96", 62, 96, 32, 8, 128, 16, "bf16", 0.088, ("uniform", 1, 3000), 3000), -1),
        (wl.DecodeConfig("ragged-96", 62, 96, 32, 8, 128, 16, "bf16", 0.088, ("uniform", 1, 3000), 3000), 64),
        (wl.DecodeConfig("gqa-f16", 63, 20, 16, 2, 64, 32, "f16", 0.125, ("uniform", 1, 5000), 5000), -2),
        (wl.DecodeConfig("one-long", 61, 1, 32, 8, 128, 16, "bf16", 0.088, ("fixed", (9000,)), 9000), -1),
    ]
    works = [wl.make_decode_workload(cfg) for cfg, _ in cases]
    need = max(pb.pa_decode_workspace_bytes(w.cfg.num_seqs, w.cfg.num_heads, w.cfg.num_kv_heads, w.cfg.head_dim,
                                            w.max_context_len, part) for w, (_, part) in zip(works, cases))
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    nc = pb.WORKSPACE_COUNTER_BYTES
    for w, (cfg, part) in zip(works, cases):
        say(f"{cfg.name} S={cfg.num_seqs} part={part}")
        d = device_case(w)
        out = fused_step(w, d, ws, part)
        torch.cuda.synchronize()
        assert int(ws[:nc].count_nonzero()) == 0, f"{cfg.name} part={part}: arrival counters left non-zero"
        seqs = list(range(0, cfg.num_seqs, max(1, cfg.num_seqs // 16)))
        check(out, oracle_out(w, seqs=seqs), f"{cfg.name} part={part}", seqs=seqs)


def test_graph_replay_matches_eager():
    """Three fused steps captured in one graph (balanced split, merged in the
    decode kernel) replay three times, with eager work and synchronizations
    between the replays, to the eager steps' output and pools bit for bit."""
    cfg = wl.DecodeConfig("graph", 64, 160, 32, 8, 128, 16, "bf16", 0.088, ("uniform", 1, 600), 600)
    w = wl.make_decode_workload(cfg)
    need = pb.pa_decode_workspace_bytes(cfg.num_seqs, 32, 8, 128, w.max_context_len, -1)
    eager, graphed = device_case(w), device_case(w)
    ws_e = torch.zeros(need, dtype=torch.uint8, device=DEV)
    ws_g = torch.zeros(need, dtype=torch.uint8, device=DEV)
    out_e = torch.empty(eager["q"].shape, dtype=torch.float32, device=DEV)
    out_g = torch.empty(eager["q"].shape, dtype=torch.float32, device=DEV)
    for _ in range(3):
        fused_step(w, eager, ws_e, out=out_e)
    torch.cuda.synchronize()
    ref = out_e.clone()
    check(ref, oracle_out(w), "eager steps")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fused_step(w, graphed, ws_g, out=out_g)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(3):
            fused_step(w, graphed, ws_g, out=out_g)
    other = device_case(w)
    ws_o = torch.zeros(need, dtype=torch.uint8, device=DEV)
    for r in range(3):
        out_g.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        say(f"  replay {r}")
        assert torch.equal(out_g, ref), f"replay {r} differs from the eager steps"
        # bit patterns: the pools hold NaN poison past the context ends
        for pool in ("kc", "vc"):
            assert torch.equal(graphed[pool].view(torch.int16), eager[pool].view(torch.int16)), f"replay {r} {pool}"
        assert int(ws_g[:pb.WORKSPACE_COUNTER_BYTES].count_nonzero()) == 0
        fused_step(w, other, ws_o)  # eager work of the program between replays
        torch.cuda.synchronize()


def test_launch_counts():
    """pa_decode_launches: one launch where the balanced split merges in the
    decode kernel (at least a quarter as many sequences as workers per KV
    head), two with the closing merge, four with the shared split's
    planning."""
    W = torch.cuda.get_device_properties(0).multi_processor_count * 4 // 8  # MFMA workers per KV head, 8 KV heads
    f = pb.pa_decode_launches
    bf16 = torch.bfloat16
    assert f(256, 32, 8, 128, 8192, -1, bf16, "auto", True) == (1 if 2 * 256 >= W else 2)
    assert f(W // 4, 32, 8, 128, 8192, -1, bf16, "auto", False) == 1
    assert f(W // 4 - 1, 32, 8, 128, 8192, -1, bf16, "auto", True) == 2
    assert f(1, 32, 8, 128, 8192, -1, bf16, "auto", False) == 2
    assert f(256, 32, 8, 128, 8192, -2, bf16, "auto", True) == 4                 # shared split
    assert f(256, 32, 8, 128, 8192, -2, torch.float32, "auto", True) == 1        # fp32 runs it as AUTO
    assert f(256, 32, 8, 128, 8192, 512, bf16, "auto", False) == 2               # fixed partitions
    assert f(256, 32, 8, 128, 8192, 0, bf16, "auto", False) == 1                 # no split
    assert f(256, 32, 8, 128, 8192, 0, bf16, "auto", True) == 2                  # no split, fused write


def test_in_kernel_merge_cut_and_empty_contexts():
    """The in-kernel path with max_context_len below the longest contexts
    (they are cut to it and their new tokens are not stored) and with
    zero-length contexts (zeros written, nothing stored): 600 sequences."""
    S, B, cut = 600, 16, 2000
    lens = mixed_lengths(S, 91)
    cfg = wl.DecodeConfig("mixed-cut", 91, S, 32, 8, 128, B, "bf16", 0.088,
                          ("fixed", tuple(int(x) for x in lens)), int(lens.max()))
    w = wl.make_decode_workload(cfg, lengths=lens)
    assert (lens > cut).sum() >= 3
    dv = device_case(w)
    empty = [5, 77, 300]
    lens_dev = lens.copy()
    lens_dev[empty] = 0
    dv["cl"] = pb.int32_to_device(lens_dev, DEV)
    need = pb.pa_decode_workspace_bytes(S, 32, 8, 128, cut, -1)
    assert pb.pa_decode_launches(S, 32, 8, 128, cut, -1, torch.bfloat16, "auto", True) == 1
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    out = torch.full(dv["q"].shape, float("nan"), dtype=torch.float32, device=DEV)
    pb.pa_write_decode(out, dv["q"], dv["kn"], dv["vn"], dv["kc"], dv["vc"], dv["bt"], dv["cl"], cfg.scale, cut,
                       workspace=ws)
    torch.cuda.synchronize()
    say(f"in-kernel merge: {int((lens > cut).sum())} contexts cut to {cut}, {len(empty)} empty")
    keep = (lens_dev > 0) & (lens_dev <= cut)
    kr, vr = oracle.write_kv(w.k_cache, w.v_cache, w.k_new[keep], w.v_new[keep], w.slot_mapping[keep], B)
    np.testing.assert_array_equal(pb.to_host(dv["kc"], "bf16").view(np.uint16), kr.view(np.uint16))
    np.testing.assert_array_equal(pb.to_host(dv["vc"], "bf16").view(np.uint16), vr.view(np.uint16))
    g = out.cpu().numpy()
    assert (g[empty] == 0).all()
    seqs = [s for s in range(S) if lens_dev[s] > 0]
    ref = oracle.decode(w.q, kr, vr, w.block_tables, np.minimum(lens_dev, cut).astype(np.int32), cfg.scale, B,
                        "bf16", seqs=seqs)
    check(out, ref, "cut and empty contexts", seqs=seqs)
    assert int(ws[:pb.WORKSPACE_COUNTER_BYTES].count_nonzero()) == 0
