"""Host logic of bench.py (CPU only): the algorithmic byte counts behind every
GB/s figure, the one-GPU guard and the counter reducer.

The byte counts are pinned to the shapes of the workloads, counted by hand:
the batch-1 MoE block streams the router [384 x 7168], the latent projection
[7168 x 7168] and nine SwiGLU experts (8 routed + 1 shared) of
3 x 2048 x 7168 bf16 weights each; the projection chain streams
[12288 x 7168] + [7168 x 8192] weights and the [7168] norm scale.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402

D, E, I, K = 7168, 384, 2048, 8


def test_moe_bytes_batch1_weights():
    cfg = synth.MOE_CONFIGS["b1"]
    weights = 2 * (E * D + D * D + 9 * 3 * I * D)
    assert weights == 900_988_928
    acts = bench.moe_bytes(cfg, 1, K) - weights
    # x, logits, ids + weights, z, routed h, shared h, y_s, y: a few tens of KB
    assert 0 < acts < 200_000


def test_moe_bytes_scale_with_active_experts():
    cfg = synth.MOE_CONFIGS["b16"]
    per_expert = 2 * 3 * I * D  # gate, up and down of one expert
    assert bench.moe_bytes(cfg, 16, 111) - bench.moe_bytes(cfg, 16, 110) == per_expert
    # the Zipf configuration also reads the fp32 router bias
    z = synth.MOE_CONFIGS["b64zipf"]
    assert bench.moe_bytes(z, 64, 50) - bench.moe_bytes(cfg, 64, 50) == 4 * E


def test_chain_bytes_weights():
    cc = synth.CHAIN_CONFIG
    weights = 2 * (12288 * D + D * 8192 + D)
    assert weights == 293_615_616
    for b in synth.CHAIN_BATCHES:
        acts = bench.chain_bytes(cc, b) - weights
        assert acts == b * (2 * D + 2 * 12288 + 2 * 8192 + 4 * D + 8 * D + 2 * D)


def test_gateup_bytes_batch1_includes_selection_and_shared_rows():
    cfg = synth.MOE_CONFIGS["b1"]
    w = 2 * K * 2 * I * D
    shared = 2 * 2 * cfg.I_s * D + 2 * D + 2 * cfg.I_s
    assert bench.gateup_bytes(cfg, 1, K) == w + 2 * D + 2 * K * I + 4 * E + 8 * K + shared
    assert bench.gateup_bytes(cfg, 16, 100) == 2 * 100 * 2 * I * D + 2 * 16 * D + 2 * 16 * K * I


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_counter_summary(tmp_path, capsys):
    run = tmp_path / "pmc_x"
    run.mkdir()
    rows = [
        ("void k3::k_sk_gemm<4, k3::SkDense>(k3::SkDense, int, int)", "MfmaUtil", "8.0"),
        ("void k3::k_sk_gemm<4, k3::SkDense>(k3::SkDense, int, int)", "MfmaUtil", "10.0"),
        ("k3::k_combine(float const*, int)", "MfmaUtil", "0"),
        ("at::native::other_kernel", "MfmaUtil", "99"),
    ]
    with open(run / "c_counter_collection.csv", "w") as f:
        f.write("Kernel_Name,Counter_Name,Counter_Value\n")
        for name, c, v in rows:
            f.write(f'"{name}",{c},{v}\n')
    assert bench.print_counter_summary(str(tmp_path)) == 0
    out = capsys.readouterr().out
    assert "| `void k3::k_sk_gemm<4, k3::SkDense>` | 2 | 9 |" in out
    assert "| `k3::k_combine` | 1 | 0 |" in out
    assert "other_kernel" not in out


def test_counter_summary_empty(tmp_path):
    assert bench.print_counter_summary(str(tmp_path)) == 2


@pytest.mark.parametrize("b", [1, 4, 64])
def test_oracle_step_counts_what_it_reads(b):
    """bench.OracleStep on the tiny layer: its byte count matches moe_bytes +
    chain_bytes for the experts its own routing picked, and it reports a
    median time on all cores and on one."""
    import types

    import numpy as np

    import oracle

    cfg = synth.MOE_CONFIGS["tiny"]
    w = synth.make_moe_weights(cfg)
    cc = synth.ChainConfig("t", d=256, n_in=384, k_o=256)
    lay = types.SimpleNamespace(moe=w, chain_w=synth.make_chain_weights(cc))
    inp = synth.make_chain_inputs(cc, b)
    o = bench.OracleStep(bench.HostWeights(lay), cfg.k, cc, inp, b, None, cfg)
    for t in bench.start_single_thread_runs([o], reps=3):
        t.join()
    o.time_all_cores(reps=3)
    rep = o.report()
    assert rep["ms_per_step"] > 0 and rep["ms_per_step_1thread"] > 0
    assert rep["runs"] == rep["runs_1thread"] == 3 and rep["cores"] >= 1
    hm = oracle.chain(inp["x"], inp["r"], lay.chain_w["w_in"], lay.chain_w["w_o"],
                      lay.chain_w["gamma"], cc.eps)["y"]
    ids, _ = oracle.topk_softmax(oracle.router_logits(hm, w["w_router"]), cfg.k)
    n_act = len(np.unique(ids))
    assert o.nbytes == bench.moe_bytes(cfg, b, n_act) + bench.chain_bytes(cc, b)
    assert rep["n_active"] == n_act


def test_trace_summary_takes_the_timed_replay(tmp_path):
    """The kernel-trace reducer picks dispatches [W + NX + K, W + NX + 2K) of
    each batch-1 step kernel as the timed region."""
    import json
    W, K = 2, 3
    names = ["void k3::k_gemv<7, 1, k3::EpiBf16>(x)", "void k3::k_oproj_gemv<8, 1>(x)",
             "void k3::k_rls_gemv<7, 1, true>(x)", "void k3::k_moe_up_b1<true, 7>(x)",
             "void k3::k_down_b1<8>(x)"]
    n_steps = W + bench.NX + 2 * K + 4  # eager, replay, then a few later steps
    t = 0
    lines = ["Kernel_Name,Start_Timestamp,End_Timestamp"]
    for i in range(n_steps):
        timed = W + bench.NX + K <= i < W + bench.NX + 2 * K
        for j, n in enumerate(names):
            d = (70_000 if timed else 90_000) if j == 3 else 10_000
            lines.append(f'"{n}",{t},{t + d}')
            t += d + 1000
    (tmp_path / "run").mkdir()
    (tmp_path / "run" / "kt_kernel_trace.csv").write_text("\n".join(lines) + "\n")
    js, md = tmp_path / "t.json", tmp_path / "t.md"
    assert bench.write_trace_summary(str(tmp_path), W, K, str(js), str(md)) == 0
    out = json.loads(js.read_text())
    assert out["dominant_timed_region_avg_us"] == 70.0
    assert out["dominant_all_dispatches_avg_us"] > 70.0
    # a step every 4 x (10 + 1) + (70 + 1) us; the span ends with the last kernel
    assert abs(out["timed_region_us_per_step"] - (K * 115.0 - 1.0) / K) < 0.01
    assert "k_moe_up_b1<true, 7>" in md.read_text()
