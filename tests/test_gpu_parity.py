"""GPU parity: every libk3dec entry point against the oracle, on the same
seeded bf16 inputs, at the tiny workload and at full size (d = 7168,
E = 384, top-8, I = 2048; projection chain 7168 -> 12288, 8192 -> 7168).

Bars: ids by the gap rule, outputs within 2e-2 * max|ref| (tests/_parity.py).
Every output of every call is compared: all tokens and all columns, at every
batch the benchmark times. Where the GPU picked another expert set inside the
1e-3 tie band, the reference continues from the GPU's set through the oracle
(ref_selection).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from _parity import assert_rel_close, check_ids, ref_selection, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _lib():
    import moe_router_topk_amd as k3
    k3.lib()
    return k3


@pytest.fixture(scope="module")
def k3():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need one")
    return _lib()


@pytest.fixture(scope="module")
def full(k3):
    """Full-size MoE weights (about 34 GB of experts) on the GPU, once."""
    cfg = synth.MOE_CONFIGS["b1"]
    w = synth.make_moe_weights(cfg, device=DEV)
    torch.cuda.synchronize()
    return cfg, w


@pytest.fixture(scope="module")
def chain_w(k3):
    w = synth.make_chain_weights(synth.CHAIN_CONFIG, device=DEV)
    torch.cuda.synchronize()
    return w


@pytest.fixture(scope="module")
def host(full):
    """Host copies of the full-size weights for the oracle, made once per
    module: the dense ones at once, each expert the first time it is named."""
    cfg, w = full
    dense = {key: w[key].cpu() for key in ("w_router", "w_lat", "w13_s", "w2_s")}
    experts = {}

    def fetch(e):
        if e not in experts:
            experts[e] = (w["w13"][e].cpu(), w["w2"][e].cpu())
        return experts[e]
    return dense, fetch


@pytest.fixture(scope="module")
def chain_host(chain_w):
    return {key: v.cpu() for key, v in chain_w.items()}


def _experts_on_host(w):
    cache = {}

    def fetch(e):
        if e not in cache:
            cache[e] = (w["w13"][e].cpu(), w["w2"][e].cpu())
        return cache[e]
    return fetch


# ---------------------------------------------------------------- router + top-k
@pytest.mark.parametrize("b,zipf", [(1, 0.0), (2, 0.0), (3, 0.0), (16, 0.0), (24, 0.0),
                                    (64, 1.1), (64, 0.0)])
def test_router_topk_full(k3, full, host, b, zipf):
    cfg, w = full
    bias = synth.zipf_router_bias(cfg.E, zipf, cfg.seed).to(DEV) if zipf else None
    x = synth.make_tokens(cfg, device=DEV, index=100 + b, b=b)
    ids, wts = k3.k3_router_topk(x, w["w_router"], bias, cfg.k)
    torch.cuda.synchronize()
    logits = oracle.router_logits(x.cpu(), host[0]["w_router"],
                                  bias.cpu() if bias is not None else None)
    _, ref_w, _ = ref_selection(ids, logits, cfg.k)
    g = wts.cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(g.sum(axis=1), 1.0, atol=1e-5)
    assert_rel_close(g, ref_w, "topk_w")
    assert (np.diff(g, axis=1) <= 1e-6).all(), "weights not in descending order"
    want = "dot2" if b <= 4 else "mfma"
    assert k3.k3_get_last_dispatch("router_topk") == want


@pytest.mark.parametrize("zipf", [0.0, 1.1])
def test_router_topk_last_workgroup_variant(k3, full, host, zipf):
    """The forced last-workgroup router (one kernel: the projection's last
    workgroup selects) gives the default two-kernel path's bits, matches the
    oracle, and leaves its counter at zero: five calls in a row on one
    workspace, on different tokens, all agree."""
    cfg, w = full
    bias = synth.zipf_router_bias(cfg.E, zipf, cfg.seed).to(DEV) if zipf else None
    nbytes = k3.workspace_size("router_topk", b=1, E=cfg.E)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    for i in range(5):
        x = synth.make_tokens(cfg, device=DEV, index=140 + i, b=1)
        ids0, wts0 = k3.k3_router_topk(x, w["w_router"], bias, cfg.k)
        k3.k3_force_variant("router_topk", "lastwg")
        try:
            ids, wts = k3.k3_router_topk(x, w["w_router"], bias, cfg.k, workspace=ws)
            torch.cuda.synchronize()
            assert k3.k3_get_last_dispatch("router_topk") == "lastwg"
        finally:
            k3.k3_force_variant("router_topk", "none")
        assert torch.equal(ids, ids0) and torch.equal(wts, wts0), f"call {i}"
        assert int(ws[:4].view(torch.int32).item()) == 0, "the counter was not reset"
        logits = oracle.router_logits(x.cpu(), host[0]["w_router"],
                                      bias.cpu() if bias is not None else None)
        _, ref_w, _ = ref_selection(ids, logits, cfg.k)
        assert_rel_close(wts.cpu().numpy().astype(np.float64), ref_w, "topk_w")


def test_router_topk_last_workgroup_variant_tiny(k3):
    """The same at the tiny workload (E = 8, one workgroup: it is its own
    last)."""
    cfg = synth.MOE_CONFIGS["tiny"]
    w = synth.make_moe_weights(cfg, device=DEV)
    x = synth.make_tokens(cfg, device=DEV, index=3, b=1)
    ids0, wts0 = k3.k3_router_topk(x, w["w_router"], None, cfg.k)
    k3.k3_force_variant("router_topk", "lastwg")
    try:
        for _ in range(3):
            ids, wts = k3.k3_router_topk(x, w["w_router"], None, cfg.k)
            torch.cuda.synchronize()
            assert torch.equal(ids, ids0) and torch.equal(wts, wts0)
    finally:
        k3.k3_force_variant("router_topk", "none")


@pytest.mark.parametrize("b", [2, 8])
def test_router_topk_ties(k3, b):
    """x = 0 makes every logit 0: ids 0..k-1 and weights 1/k (row engine at
    2 tokens, the MFMA pass with its finish-and-select kernel at 8)."""
    x = torch.zeros((b, 256), dtype=torch.bfloat16, device=DEV)
    wr = synth.uniform_bf16((8, 256), 0.1, 0, "tie", device=DEV)
    ids, wts = k3.k3_router_topk(x, wr, None, 3)
    torch.cuda.synchronize()
    assert ids.cpu().tolist() == [[0, 1, 2]] * b
    np.testing.assert_allclose(wts.cpu().numpy(), 1 / 3, rtol=1e-6)


@pytest.mark.parametrize("b", [4, 8, 33])
def test_router_topk_k_equals_E(k3, b):
    cfg = synth.MOE_CONFIGS["tiny"]
    w = synth.make_moe_weights(cfg, device=DEV)
    x = synth.make_tokens(cfg, device=DEV, b=b)
    ids, wts = k3.k3_router_topk(x, w["w_router"], None, cfg.E)
    torch.cuda.synchronize()
    logits = oracle.router_logits(x.cpu(), w["w_router"].cpu())
    ref_ids, ref_w = oracle.topk_softmax(logits, cfg.E)
    check_ids(ids, ref_ids, logits, cfg.E)
    assert_rel_close(wts.cpu(), ref_w, "topk_w")


@pytest.mark.parametrize("b", [1, 3, 8, 40])
def test_router_topk_many_experts(k3, b):
    """E = 1000 experts (near the 1024 limit, not a multiple of the wave),
    k = 16, with a bias: every engine's selection against the oracle."""
    E, d, k = 1000, 512, 16
    wr = synth.uniform_bf16((E, d), math.sqrt(3.0 / d), 0, "many_wr", device=DEV)
    bias = synth.zipf_router_bias(E, 1.1, 0).to(DEV)
    x = synth.randn_bf16((b, d), 1.0, 0, "many_x", b, device=DEV)
    ids, wts = k3.k3_router_topk(x, wr, bias, k)
    torch.cuda.synchronize()
    logits = oracle.router_logits(x.cpu(), wr.cpu(), bias.cpu())
    _, ref_w, _ = ref_selection(ids, logits, k)
    assert_rel_close(wts.cpu().numpy(), ref_w, "topk_w")


@pytest.mark.parametrize("b,zipf", [(1, 0.0), (2, 0.0), (4, 1.1), (8, 0.0), (16, 0.0),
                                    (24, 0.0), (40, 0.0), (64, 1.1)])
def test_router_topk_latent_full(k3, full, host, b, zipf):
    """The fused router + latent pass: ids and weights as k3_router_topk, z as
    k3_proj_skinny, at full size (dot2 up to 4 tokens, MFMA above). Bit for
    bit where the separate latent projection takes the fused pass's summation
    order; at 5-32 tokens it takes the whole-K pass (1024-wide K slices
    instead of K ranges), and the two z agree to rounding."""
    cfg, w = full
    bias = synth.zipf_router_bias(cfg.E, zipf, cfg.seed).to(DEV) if zipf else None
    x = synth.make_tokens(cfg, device=DEV, index=150 + b, b=b)
    ids, wts, z = k3.k3_router_topk_latent(x, w["w_router"], bias, cfg.k, w["w_lat"])
    torch.cuda.synchronize()
    assert k3.k3_get_last_dispatch("router_latent") == ("dot2" if b <= 4 else "mfma")
    logits = oracle.router_logits(x.cpu(), host[0]["w_router"],
                                  bias.cpu() if bias is not None else None)
    _, ref_w, _ = ref_selection(ids, logits, cfg.k)
    assert_rel_close(wts.cpu().numpy(), ref_w, "topk_w")
    assert_rel_close(z.cpu(), oracle.linear(x.cpu(), host[0]["w_lat"]), "z")
    # the same bits as the two separate calls
    ids2, wts2 = k3.k3_router_topk(x, w["w_router"], bias, cfg.k)
    z2 = k3.k3_proj_skinny(x, w["w_lat"])
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and torch.equal(wts, wts2)
    if b > 4 and k3.k3_get_last_dispatch("dense_pass") == "wholek":
        # fp32 sums in two orders, each rounded to bf16: at most a couple of
        # bf16 units apart (2^-8 relative each)
        assert_rel_close(z2.cpu(), z.float().cpu(), "z, separate against fused", tol=8e-3)
    else:
        assert torch.equal(z, z2)


def test_router_topk_latent_tiny_repeated(k3):
    """Tiny workload, several calls in a row on one workspace (the counter
    resets) and E not a multiple of the wave count."""
    cfg = synth.MOE_CONFIGS["tiny"]
    w = synth.make_moe_weights(cfg, device=DEV)
    for b in (1, 3, 4, 1):
        x = synth.make_tokens(cfg, device=DEV, index=60 + b, b=b)
        ids, wts, z = k3.k3_router_topk_latent(x, w["w_router"], None, cfg.k, w["w_lat"])
        torch.cuda.synchronize()
        logits = oracle.router_logits(x.cpu(), w["w_router"].cpu())
        ref_ids, ref_w = oracle.topk_softmax(logits, cfg.k)
        check_ids(ids, ref_ids, logits, cfg.k)
        assert_rel_close(wts.cpu(), ref_w, "topk_w")
        assert_rel_close(z.cpu(), oracle.linear(x.cpu(), w["w_lat"].cpu()), "z")


# ---------------------------------------------------------------- skinny projection
def dense_pass_for(b, K):
    """The MFMA pass a single dense projection takes above four tokens."""
    if 5 <= b <= 32 and K % 1024 == 0 and K // 1024 in (7, 8):
        return "wholek"
    return "resident" if b <= 32 else "splitk"


@pytest.mark.parametrize("b", [1, 2, 3, 4, 5, 8, 9, 16, 17, 24, 32, 33, 40, 48, 56, 64])
def test_proj_skinny_latent(k3, full, host, b):
    cfg, w = full
    x = synth.make_tokens(cfg, device=DEV, index=200 + b, b=b)
    y = k3.k3_proj_skinny(x, w["w_lat"])
    torch.cuda.synchronize()
    assert_rel_close(y.cpu(), oracle.linear(x.cpu(), host[0]["w_lat"]), "z")
    assert k3.k3_get_last_dispatch("proj_skinny") == ("dot2" if b <= 4 else "mfma")
    if b > 4:
        assert k3.k3_get_last_dispatch("dense_pass") == dense_pass_for(b, cfg.d)


@pytest.mark.parametrize("variant", ["dot2", "mfma"])
@pytest.mark.parametrize("b,K,N", [(1, 256, 256), (2, 128, 40), (4, 1024, 1000), (3, 896, 33),
                                   (4, 8192, 77), (1, 2056, 5), (8, 1024, 1000), (7, 896, 33)])
def test_proj_skinny_ragged(k3, variant, b, K, N):
    """Both engines on small ragged shapes (N not a multiple of 16, few rows,
    K not a multiple of the 512-element row chunk)."""
    if variant == "mfma" and K % 128:
        pytest.skip("MFMA engine needs K % 128 == 0")
    if variant == "dot2" and b > 4:
        pytest.skip("dot2 engine takes at most 4 tokens")
    x = synth.randn_bf16((b, K), 1.0, 7, "rag_x", K * 100 + N, device=DEV)
    W = synth.randn_bf16((N, K), 1 / math.sqrt(K), 7, "rag_w", K * 100 + N, device=DEV)
    k3.k3_force_variant("proj_skinny", variant)
    try:
        y = k3.k3_proj_skinny(x, W)
        torch.cuda.synchronize()
        assert k3.k3_get_last_dispatch("proj_skinny") == variant
    finally:
        k3.k3_force_variant("proj_skinny", "none")
    assert_rel_close(y.cpu(), oracle.linear(x.cpu(), W.cpu()), "y")


@pytest.mark.parametrize("b", [1, 2, 3, 4])
@pytest.mark.parametrize("K,N", [(64, 24), (128, 40), (192, 17), (320, 9), (7168, 13),
                                 (8192, 1000)])
def test_row_engine_short_and_uneven_rows(k3, K, N, b):
    """1..4 tokens on the 8-row engine: K-quarters that are empty (K < 256)
    or uneven (K / 64 not a multiple of 4), partial 8-row groups, and fewer
    rows than workgroups; token rows ldx apart."""
    xb = synth.randn_bf16((b, K + 64), 1.0, 9, "b1e_x", K * 100 + N + b, device=DEV)
    x = xb[:, 32:32 + K]
    W = synth.randn_bf16((N, K), 1 / math.sqrt(K), 9, "b1e_w", K * 100 + N, device=DEV)
    y = k3.k3_proj_skinny(x, W)
    torch.cuda.synchronize()
    assert k3.k3_get_last_dispatch("proj_skinny") == "dot2"
    assert_rel_close(y.cpu(), oracle.linear(x.cpu(), W.cpu()), "y")
    # the o-projection with residual and RMSNorm on the same shapes (d = N)
    r = synth.randn_bf16((b, N), 1.0, 9, "b1e_r", K * 100 + N + b, device=DEV)
    g = (synth.randn_bf16((N,), 0.1, 9, "b1e_g", K * 100 + N, device=DEV).float() + 1).to(
        torch.bfloat16)
    r0 = r.clone()
    if N % 8 == 0:
        yn = k3.k3_oproj_residual(x, W, r, g, 1e-6)
        torch.cuda.synchronize()
        h_ref, y_ref = oracle.oproj_residual_rmsnorm(x.cpu(), W.cpu(), r0.cpu(), g.cpu(), 1e-6)
        assert_rel_close(r.cpu(), h_ref, "h")
        assert_rel_close(yn.cpu(), y_ref, "y_norm")


@pytest.mark.parametrize("b", sorted(set(synth.CHAIN_BATCHES)
                                    | {5, 6, 7, 9, 12, 15, 17, 20, 24, 31, 33, 40, 48, 56}))
def test_proj_skinny_chain_in(k3, chain_w, chain_host, b):
    """The attention input projection 7168 -> 12288 at every chain batch the
    benchmark times, the verify batches 8 r and 5-7, 9, 12, 15, 17, 20, 31 and
    33 tokens (the whole-K pass covers 5-32: the slice staged whole up to 8
    tokens, in halves up to 16, in quarters with two token blocks up to 32);
    every output."""
    inp = synth.make_chain_inputs(synth.CHAIN_CONFIG, b, device=DEV, index=300 + b)
    q = k3.k3_proj_skinny(inp["x"], chain_w["w_in"])
    torch.cuda.synchronize()
    assert_rel_close(q.cpu(), oracle.linear(inp["x"].cpu(), chain_host["w_in"]), "q")
    assert k3.k3_get_last_dispatch("proj_skinny") == ("dot2" if b <= 4 else "mfma")
    if b > 4:
        assert k3.k3_get_last_dispatch("dense_pass") == dense_pass_for(b, synth.CHAIN_CONFIG.d)


@pytest.mark.parametrize("b,K,N", [(5, 7168, 12248), (11, 8192, 5000), (16, 7168, 16384),
                                   (9, 8192, 4104), (13, 7168, 4100), (8, 8192, 7168),
                                   (17, 8192, 7168), (23, 7168, 12248), (29, 8192, 5000),
                                   (32, 7168, 16384), (19, 7168, 4100), (32, 8192, 4104)])
def test_whole_k_pass_shapes(k3, b, K, N):
    """The whole-K pass at the edges of its shapes: rows per workgroup from
    17 to 64 (two to four 16-row tiles, the last short), N not a multiple of
    16 (the last workgroup's rows partial), seven and eight K slices, the
    slice staged whole, in halves and in quarters (17-32 tokens: two token
    blocks, the second partial below 32), x and y as column slices of wider
    buffers; then the o-projection form (residual add) on the same shape."""
    xb = synth.randn_bf16((b, K + 32), 1.0, 11, "wk_x", K * 100 + N + b, device=DEV)
    x = xb[:, 32:]
    W = synth.randn_bf16((N, K), 1 / math.sqrt(K), 11, "wk_w", K * 100 + N, device=DEV)
    yb = torch.zeros((b, N + 24), dtype=torch.bfloat16, device=DEV)
    y = yb[:, :N]
    k3.k3_proj_skinny(x, W, y=y)
    torch.cuda.synchronize()
    assert k3.k3_get_last_dispatch("dense_pass") == "wholek"
    assert_rel_close(y.cpu(), oracle.linear(x.cpu(), W.cpu()), "y")
    assert (yb[:, N:] == 0).all()
    if N % 8 == 0 and N <= 8192:  # the o-projection's width limits
        r = synth.randn_bf16((b, N), 1.0, 11, "wk_r", K * 100 + N + b, device=DEV)
        g = (synth.randn_bf16((N,), 0.1, 11, "wk_g", N, device=DEV).float() + 1).to(
            torch.bfloat16)
        r0 = r.clone()
        yn = k3.k3_oproj_residual(x, W, r, g, 1e-6)
        torch.cuda.synchronize()
        assert k3.k3_get_last_dispatch("dense_pass") == "wholek"
        h_ref, y_ref = oracle.oproj_residual_rmsnorm(x.cpu(), W.cpu(), r0.cpu(), g.cpu(), 1e-6)
        assert_rel_close(r.cpu(), h_ref, "h")
        assert_rel_close(yn.cpu(), y_ref, "y_norm")


@pytest.mark.parametrize("b", [3, 20])
def test_proj_skinny_strided_output(k3, chain_w, chain_host, b):
    """x and y as column slices of wider buffers (row strides > width), on
    the 8-row engine (3 tokens) and the MFMA engine (20)."""
    w = chain_w
    xb = synth.randn_bf16((b, 7168 + 64), 1.0, 0, "strided_x", b, device=DEV)
    x = xb[:, 64:]
    yb = torch.zeros((b, 12288 + 128), dtype=torch.bfloat16, device=DEV)
    y = yb[:, :12288]
    k3.k3_proj_skinny(x, w["w_in"], y=y)
    torch.cuda.synchronize()
    assert_rel_close(y.cpu(), oracle.linear(x.cpu(), chain_host["w_in"]), "q")
    assert (yb[:, 12288:] == 0).all()


# ---------------------------------------------------------------- per-GPU TP8 shares
@pytest.fixture(scope="module")
def shard(k3):
    """One GPU's share of the experts under tensor parallelism over 8 GPUs
    (I = I_s = 256), with the router and latent rows whole."""
    cfg = synth.MOE_CONFIGS["tp8_shard"]
    w = synth.make_moe_weights(cfg, device=DEV)
    torch.cuda.synchronize()
    return cfg, w, _experts_on_host(w)


@pytest.mark.parametrize("b,zipf", [(1, 0.0), (3, 0.0), (16, 0.0), (64, 1.1)])
def test_moe_experts_tp8_shard(k3, shard, b, zipf):
    """Routed experts at one GPU's TP8 share (gate/up [512 x 7168], down
    [7168 x 256] per expert; the all-reduce of y is not run): every token
    against the oracle, on the engine the batch calls for."""
    cfg, w, fetch = shard
    x, z, ids, wts, y_add, y = _routed_case(k3, cfg, w, b, zipf, 600 + b)
    assert k3.k3_get_last_dispatch("expert_engine") == _engine(b)
    ref = oracle.moe_experts(z.cpu(), ids.cpu().numpy(), wts.cpu().numpy(), fetch, cfg.E,
                             y_add=y_add.cpu())
    assert_rel_close(y.cpu(), ref, "y")


@pytest.mark.parametrize("b", [1, 4, 16, 64])
def test_shared_expert_tp8_shard(k3, shard, b):
    cfg, w, _ = shard
    x = synth.make_tokens(cfg, device=DEV, index=620 + b, b=b)
    y_s = k3.k3_shared_expert(x, w["w13_s"], w["w2_s"])
    torch.cuda.synchronize()
    ref = oracle.shared_expert(x.cpu(), w["w13_s"].cpu(), w["w2_s"].cpu())
    assert_rel_close(y_s.cpu(), ref, "y_s")


@pytest.mark.parametrize("b", [1, 8, 64])
def test_chain_projections_tp8_shard(k3, chain_w, chain_host, b):
    """The chain's projections at one GPU's TP8 share: the input projection's
    rows split (1536 x 7168) and the o-projection's K split (7168 x 1024;
    the all-reduce that would precede the norm is not run): every output."""
    cc = synth.CHAIN_CONFIG
    inp = synth.make_chain_inputs(cc, b, device=DEV, index=640 + b)
    q = k3.k3_proj_skinny(inp["x"], chain_w["w_in"][:1536])
    w_o = chain_w["w_o"][:, :1024].contiguous()
    a = synth.randn_bf16((b, 1024), 1.0, 0, "tp8_a", b, device=DEV)
    r = synth.randn_bf16((b, cc.d), 1.0, 0, "tp8_r", b, device=DEV)
    r_in = r.clone()
    y = k3.k3_oproj_residual(a, w_o, r, chain_w["gamma"], cc.eps)
    torch.cuda.synchronize()
    assert_rel_close(q.cpu(), oracle.linear(inp["x"].cpu(), chain_host["w_in"][:1536]), "q")
    h_ref, y_ref = oracle.oproj_residual_rmsnorm(a.cpu(), w_o.cpu(), r_in.cpu(),
                                                 chain_host["gamma"], cc.eps)
    assert_rel_close(r.cpu(), h_ref, "h")
    assert_rel_close(y.cpu(), y_ref, "y_norm")


# ---------------------------------------------------------------- shared expert
@pytest.mark.parametrize("b", [1, 2, 4, 16, 40, 64])
def test_shared_expert_full(k3, full, host, b):
    cfg, w = full
    x = synth.make_tokens(cfg, device=DEV, index=300 + b, b=b)
    y_s = k3.k3_shared_expert(x, w["w13_s"], w["w2_s"])
    torch.cuda.synchronize()
    ref = oracle.shared_expert(x.cpu(), host[0]["w13_s"], host[0]["w2_s"])
    assert_rel_close(y_s.cpu(), ref, "y_s")
    assert k3.k3_get_last_dispatch("shared_expert") == ("dot2" if b <= 4 else "mfma")


@pytest.mark.parametrize("cu_budget", [1, 8, 32])
def test_shared_expert_cu_budget(k3, full, cu_budget):
    """A CU budget changes the grid, not the result bits."""
    cfg, w = full
    x = synth.make_tokens(cfg, device=DEV, index=77, b=3)
    a = k3.k3_shared_expert(x, w["w13_s"], w["w2_s"]).clone()
    bb = k3.k3_shared_expert(x, w["w13_s"], w["w2_s"], cu_budget=cu_budget)
    torch.cuda.synchronize()
    assert torch.equal(a, bb)


# ---------------------------------------------------------------- routed experts
def _routed_case(k3, cfg, w, b, zipf, index, ids_override=None):
    bias = synth.zipf_router_bias(cfg.E, zipf, cfg.seed).to(DEV) if zipf else None
    x = synth.make_tokens(cfg, device=DEV, index=index, b=b)
    ids, wts = k3.k3_router_topk(x, w["w_router"], bias, cfg.k)
    if ids_override is not None:
        ids = ids_override
    z = k3.k3_proj_skinny(x, w["w_lat"])
    y_add = synth.randn_bf16((b, cfg.d), 0.05, 9, "y_add", index, device=DEV).float()
    y = k3.k3_moe_experts(z, ids, wts, w["w13"], w["w2"], y_add=y_add)
    torch.cuda.synchronize()
    return x, z, ids, wts, y_add, y


def _engine(b):
    return "dot2" if b <= 4 else "mfma"


@pytest.mark.parametrize("b,zipf", [(1, 0.0), (2, 0.0), (3, 0.0), (4, 0.0), (8, 0.0),
                                    (16, 0.0), (24, 0.0), (32, 0.0), (40, 0.0), (48, 0.0),
                                    (56, 0.0), (64, 0.0), (64, 1.1)])
def test_moe_experts_full(k3, full, host, b, zipf):
    """Every token's y against the oracle on the GPU's own ids and weights;
    the expert engine is the one the batch calls for (dot2 rows up to 4
    tokens, MFMA tiles above)."""
    cfg, w = full
    x, z, ids, wts, y_add, y = _routed_case(k3, cfg, w, b, zipf, 400 + b)
    assert k3.k3_get_last_dispatch("moe_experts") == "grouped"
    assert k3.k3_get_last_dispatch("expert_engine") == _engine(b)
    counts = np.bincount(ids.cpu().numpy().ravel(), minlength=cfg.E)
    print(f"b={b} zipf={zipf}: active experts {int((counts > 0).sum())}, "
          f"max tokens/expert {int(counts.max())}", flush=True)
    ref = oracle.moe_experts(z.cpu(), ids.cpu().numpy(), wts.cpu().numpy(), host[1], cfg.E,
                             y_add=y_add.cpu())
    assert_rel_close(y.cpu(), ref, "y")


def test_moe_experts_hot_expert_tiles(k3, full, host):
    """All 64 tokens on the same 8 experts: four 16-token MFMA tiles each,
    on the MFMA engine; every token compared."""
    cfg, w = full
    b = 64
    ids = torch.tensor([[3, 17, 42, 99, 100, 255, 300, 383]] * b, dtype=torch.int32, device=DEV)
    ids = ids[:, torch.randperm(8, generator=torch.Generator().manual_seed(1))].contiguous()
    x, z, _, wts, y_add, y = _routed_case(k3, cfg, w, b, 0.0, 500, ids_override=ids)
    assert k3.k3_get_last_dispatch("expert_engine") == "mfma"
    ref = oracle.moe_experts(z.cpu(), ids.cpu().numpy(), wts.cpu().numpy(), host[1], cfg.E,
                             y_add=y_add.cpu())
    assert_rel_close(y.cpu(), ref, "y")


@pytest.mark.parametrize("b", [2, 3, 4])
def test_moe_experts_forced_mfma_small_batch(k3, full, host, b):
    """Batches 2-4 forced onto the MFMA tiles (light experts only, 16-token
    tiles with 1-4 live rows): the same outputs as the oracle."""
    cfg, w = full
    k3.k3_force_variant("expert_engine", "mfma")
    try:
        x, z, ids, wts, y_add, y = _routed_case(k3, cfg, w, b, 0.0, 450 + b)
        assert k3.k3_get_last_dispatch("expert_engine") == "mfma"
    finally:
        k3.k3_force_variant("expert_engine", "none")
    ref = oracle.moe_experts(z.cpu(), ids.cpu().numpy(), wts.cpu().numpy(), host[1], cfg.E,
                             y_add=y_add.cpu())
    assert_rel_close(y.cpu(), ref, "y")


def test_moe_experts_forced_engine_rejected(k3, full):
    """A forced engine that cannot run the batch fails loudly, launching
    nothing: MFMA at batch 1 (no permutation there), dot2 above 4 tokens."""
    cfg, w = full
    for variant, b in (("mfma", 1), ("dot2", 5)):
        x = synth.make_tokens(cfg, device=DEV, index=460 + b, b=b)
        z = k3.k3_proj_skinny(x, w["w_lat"])
        ids, wts = k3.k3_router_topk(x, w["w_router"], None, cfg.k)
        k3.k3_force_variant("expert_engine", variant)
        try:
            with pytest.raises(k3.K3Error) as ei:
                k3.k3_moe_experts(z, ids, wts, w["w13"], w["w2"])
            assert ei.value.status == -2
        finally:
            k3.k3_force_variant("expert_engine", "none")


def test_moe_experts_deterministic(k3, full):
    cfg, w = full
    a = _routed_case(k3, cfg, w, 16, 0.0, 600)[-1].clone()
    bb = _routed_case(k3, cfg, w, 16, 0.0, 600)[-1]
    assert torch.equal(a, bb)


@pytest.mark.parametrize("b,zipf", [(24, 0.0), (48, 0.0), (64, 1.1)])
def test_moe_experts_schedule_does_not_change_bits(k3, full, b, zipf):
    """Which workgroup takes which expert item does not change any output:
    the full-device launch (two workgroups per compute unit, slot shares and
    XCD-grouped rounds above 16 tokens) against a budget of all but one
    compute unit (an odd grid: plain round-robin items), bit for bit."""
    cfg, w = full
    _, z, ids, wts, y_add, y = _routed_case(k3, cfg, w, b, zipf, 650 + b)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    y2 = k3.k3_moe_experts(z, ids, wts, w["w13"], w["w2"], y_add=y_add, cu_budget=cus - 1)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)


def test_moe_experts_b1_invalid_id_dropped(k3):
    """Batch 1 (slots are experts, no permutation): an id outside [0, E)
    contributes nothing."""
    cfg = synth.MOE_CONFIGS["tiny"]
    w = synth.make_moe_weights(cfg, device=DEV)
    x = synth.make_tokens(cfg, device=DEV, b=1)
    z = k3.k3_proj_skinny(x, w["w_lat"])
    ids = torch.tensor([[6, 99]], dtype=torch.int32, device=DEV)
    wts = torch.tensor([[0.625, 0.375]], dtype=torch.float32, device=DEV)
    y = k3.k3_moe_experts(z, ids, wts, w["w13"], w["w2"])
    torch.cuda.synchronize()
    ref = oracle.moe_experts(z.cpu(), np.array([[6, 6]], np.int32), np.array([[0.625, 0.0]]),
                             _experts_on_host(w), cfg.E)
    assert_rel_close(y.cpu(), ref, "y")


def test_moe_experts_b1_generic_down(k3):
    """Batch 1 with I > 2048: the generic down kernel and the ordered combine
    (slot positions from the ids) instead of the row-owning kernel."""
    E, d, I, k = 6, 256, 2176, 3
    w13 = synth.randn_bf16((E, 2 * I, d), 1 / 16, 2, "g_w13", device=DEV)
    w2 = synth.randn_bf16((E, d, I), 1 / math.sqrt(I), 2, "g_w2", device=DEV)
    z = synth.randn_bf16((1, d), 1.0, 2, "g_z", device=DEV)
    ids = torch.tensor([[4, 1, 5]], dtype=torch.int32, device=DEV)
    wts = torch.tensor([[0.5, 0.3, 0.2]], dtype=torch.float32, device=DEV)
    y_add = synth.randn_bf16((1, d), 0.1, 2, "g_ya", device=DEV).float()
    y = k3.k3_moe_experts(z, ids, wts, w13, w2, y_add=y_add)
    torch.cuda.synchronize()
    fn = lambda e: (w13[e].cpu(), w2[e].cpu())  # noqa: E731
    ref = oracle.moe_experts(z.cpu(), ids.cpu().numpy(), wts.cpu().numpy(), fn, E,
                             y_add=y_add.cpu())
    assert_rel_close(y.cpu(), ref, "y")


@pytest.mark.parametrize("b", [3, 4, 5, 8])
def test_moe_experts_light_and_heavy_lists(k3, b):
    """Tokens forced onto few experts so some have more than 4 tokens (MFMA
    tiles) and some at most 4 (dot2 rows), at the tiny workload."""
    cfg = synth.MOE_CONFIGS["tiny"]
    w = synth.make_moe_weights(cfg, device=DEV)
    x = synth.make_tokens(cfg, device=DEV, index=40 + b, b=b)
    z = k3.k3_proj_skinny(x, w["w_lat"])
    ids = torch.tensor([[3, t % cfg.E] if t % cfg.E != 3 else [3, 0] for t in range(b)],
                       dtype=torch.int32, device=DEV)
    wts = torch.full((b, 2), 0.5, dtype=torch.float32, device=DEV)
    y_add = synth.randn_bf16((b, cfg.d), 0.1, 3, "ya_lh", b, device=DEV).float()
    y = k3.k3_moe_experts(z, ids, wts, w["w13"], w["w2"], y_add=y_add)
    torch.cuda.synchronize()
    ref = oracle.moe_experts(z.cpu(), ids.cpu().numpy(), wts.cpu().numpy(), _experts_on_host(w),
                             cfg.E, y_add=y_add.cpu())
    assert_rel_close(y.cpu(), ref, "y")


def test_workspace_reuse_across_shapes(k3, full, chain_w):
    """A workspace needs no initialisation and keeps no state: filled with
    NaN bit patterns, then reused by calls of other shapes, it gives the bits
    a fresh workspace gives (the split-K partial sums of the MFMA variants
    are written in full before they are read)."""
    cfg, w = full
    for b in (2, 16):
        x = synth.make_tokens(cfg, device=DEV, index=900 + b, b=b)
        ref = k3.k3_router_topk(x, w["w_router"], None, cfg.k)
        ws = torch.full((k3.workspace_size("router_topk", b=16, E=cfg.E),), 0xFF,
                        dtype=torch.uint8, device=DEV)
        xb = synth.make_tokens(cfg, device=DEV, index=901, b=1)
        k3.k3_router_topk(xb, w["w_router"], None, cfg.k, workspace=ws)  # another shape first
        for rep in range(2):
            ids, wts = k3.k3_router_topk(x, w["w_router"], None, cfg.k, workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(ids, ref[0]) and torch.equal(wts, ref[1])
    cc = synth.CHAIN_CONFIG
    for b in (1, 8):
        a = synth.randn_bf16((b, cc.k_o), 1.0, 0, "cnt_a", device=DEV)
        r0 = synth.randn_bf16((b, cc.d), 1.0, 0, "cnt_r", device=DEV)
        r_ref = r0.clone()
        y_ref = k3.k3_oproj_residual(a, chain_w["w_o"], r_ref, chain_w["gamma"], cc.eps)
        wso = torch.full((k3.workspace_size("oproj_residual", b=8, K=cc.k_o, d=cc.d),), 0xFF,
                         dtype=torch.uint8, device=DEV)
        for rep in range(2):
            r = r0.clone()
            y = k3.k3_oproj_residual(a, chain_w["w_o"], r, chain_w["gamma"], cc.eps,
                                     workspace=wso)
            torch.cuda.synchronize()
            assert torch.equal(y, y_ref) and torch.equal(r, r_ref)


def test_moe_experts_invalid_ids_dropped(k3):
    """Ids outside [0, E) contribute nothing (and read no memory)."""
    cfg = synth.MOE_CONFIGS["tiny"]
    w = synth.make_moe_weights(cfg, device=DEV)
    x = synth.make_tokens(cfg, device=DEV, b=2)
    z = k3.k3_proj_skinny(x, w["w_lat"])
    ids = torch.tensor([[1, -1], [8, 5]], dtype=torch.int32, device=DEV)
    wts = torch.tensor([[0.5, 0.5], [0.25, 0.75]], dtype=torch.float32, device=DEV)
    y = k3.k3_moe_experts(z, ids, wts, w["w13"], w["w2"])
    torch.cuda.synchronize()
    ref = oracle.moe_experts(z.cpu(), np.array([[1, 1], [5, 5]], np.int32),
                             np.array([[0.5, 0.0], [0.0, 0.75]]), _experts_on_host(w), cfg.E)
    assert_rel_close(y.cpu(), ref, "y")


# ---------------------------------------------------------------- o-proj + residual + norm
@pytest.mark.parametrize("b", [1, 2, 3, 4, 5, 6, 7, 8, 9, 13, 16, 17, 24, 32, 40, 48, 56, 64])
def test_oproj_residual_full(k3, chain_w, chain_host, b):
    w = chain_w
    cc = synth.CHAIN_CONFIG
    a_full = synth.randn_bf16((b, cc.n_in), 1.0, 0, "oproj_a", b, device=DEV)
    a = a_full[:, :cc.k_o]
    r = synth.randn_bf16((b, cc.d), 1.0, 0, "oproj_r", b, device=DEV)
    r_in = r.clone()
    y = k3.k3_oproj_residual(a, w["w_o"], r, w["gamma"], cc.eps)
    torch.cuda.synchronize()
    h_ref, y_ref = oracle.oproj_residual_rmsnorm(a.cpu(), chain_host["w_o"], r_in.cpu(),
                                                 chain_host["gamma"], cc.eps)
    assert_rel_close(r.cpu(), h_ref, "h")
    assert_rel_close(y.cpu(), y_ref, "y_norm")
    assert k3.k3_get_last_dispatch("oproj_residual") == ("dot2" if b <= 4 else "mfma")
    if b > 4:
        assert k3.k3_get_last_dispatch("dense_pass") == dense_pass_for(b, cc.k_o)


def test_oproj_residual_identity_norm(k3):
    """W_o = 0: h = r bit for bit, and y = RMSNorm(r) * gamma."""
    d, K = 256, 128
    a = synth.randn_bf16((3, K), 1.0, 1, "idn_a", device=DEV)
    wo = torch.zeros((d, K), dtype=torch.bfloat16, device=DEV)
    r = synth.randn_bf16((3, d), 1.0, 1, "idn_r", device=DEV)
    g = synth.randn_bf16((d,), 0.1, 1, "idn_g", device=DEV) + 1
    r0 = r.clone()
    y = k3.k3_oproj_residual(a, wo, r, g.to(torch.bfloat16), 1e-6)
    torch.cuda.synchronize()
    assert torch.equal(r, r0)
    _, yr = oracle.oproj_residual_rmsnorm(a.cpu(), wo.cpu(), r0.cpu(), g.to(torch.bfloat16).cpu(),
                                          1e-6)
    assert_rel_close(y.cpu(), yr, "y_norm")


# ---------------------------------------------------------------- prefetch
def test_prefetch_reads_only(k3):
    t = synth.randn_bf16((1 << 20,), 1.0, 0, "pf", device=DEV)
    t0 = t.clone()
    k3.k3_prefetch(t, cu_budget=16)
    k3.k3_prefetch(t, nbytes=16)
    k3.k3_prefetch(t, nbytes=0)
    torch.cuda.synchronize()
    assert torch.equal(t, t0)
    assert k3.k3_get_last_dispatch("prefetch") == "stream"


def test_stream_read_reads_only(k3):
    t = synth.randn_bf16((1 << 20,), 1.0, 0, "sr", device=DEV)
    t0 = t.clone()
    k3.k3_stream_read(t)
    k3.k3_stream_read(t, nbytes=16)
    k3.k3_stream_read(t, nbytes=0)
    torch.cuda.synchronize()
    assert torch.equal(t, t0)
    with pytest.raises(k3.K3Error):
        k3.k3_stream_read(t, nbytes=24)


# ---------------------------------------------------------------- whole block / layer
def test_tiny_layer_end_to_end(k3):
    from moe_router_topk_amd.layer import DecodeLayer
    cfg = synth.MOE_CONFIGS["tiny"]
    w = synth.make_moe_weights(cfg, device=DEV)
    layer = DecodeLayer(w, cfg.k, b_max=4)
    for b in (1, 4):
        x = synth.make_tokens(cfg, device=DEV, index=b, b=b)
        y = layer.moe_block(x)
        torch.cuda.synchronize()
        wc = {key: (v.cpu() if v is not None else None) for key, v in w.items()}
        ref = oracle.moe_block(x.cpu(), wc, cfg.k)
        check_ids(layer.ids[:b], ref["ids"], ref["logits"], cfg.k)
        assert_rel_close(layer.z[:b].cpu(), ref["z"], "z")
        assert_rel_close(layer.y_s[:b].cpu(), ref["y_s"], "y_s")
        assert_rel_close(y.cpu(), ref["y"], "y")


# the batches the benchmark times the block and the layer step at: 1, 2, 4,
# the verify batches 8 r (r = 1..8) with uniform routing, and 64 with the
# Zipf(1.1) router bias
BLOCK_CASES = [(1, 0.0), (2, 0.0), (4, 0.0), (8, 0.0), (16, 0.0), (24, 0.0), (32, 0.0),
               (40, 0.0), (48, 0.0), (56, 0.0), (64, 0.0), (64, 1.1)]


def _block_reference(xh, dense, fetch, bias, gpu_ids, k, E):
    """The oracle's MoE block on the bf16 block input xh (host), carrying
    fp64 intermediates, continued from the GPU's expert set inside the tie
    band: (y, z, y_s, differing tokens)."""
    logits = oracle.router_logits(xh, dense["w_router"], bias)
    ids, wt, differ = ref_selection(gpu_ids, logits, k)
    z = oracle.linear(xh, dense["w_lat"])
    y_s = oracle.shared_expert(xh, dense["w13_s"], dense["w2_s"])
    y = oracle.moe_experts(z, ids, wt, fetch, E, y_add=y_s)
    return y, z, y_s, differ


@pytest.mark.parametrize("b,zipf", BLOCK_CASES)
def test_moe_block_end_to_end_full(k3, full, host, b, zipf):
    """The fused single-stream block (k3_moe_block, as the benchmark times
    it) against the oracle carrying fp64 intermediates: every token of z,
    y_s and y, and the weights."""
    from moe_router_topk_amd.layer import DecodeLayer
    cfg, w = full
    w = dict(w)
    w["bias"] = synth.zipf_router_bias(cfg.E, zipf, cfg.seed).to(DEV) if zipf else None
    layer = DecodeLayer(w, cfg.k, b_max=b)
    x = synth.make_tokens(cfg, device=DEV, index=700 + b, b=b)
    y = layer.moe_block(x)
    torch.cuda.synchronize()
    assert k3.k3_get_last_dispatch("expert_engine") == _engine(b)
    bias = w["bias"].cpu() if zipf else None
    ref, z, y_s, differ = _block_reference(x.cpu(), host[0], host[1], bias, layer.ids[:b],
                                           cfg.k, cfg.E)
    if differ:
        print(f"b={b}: tokens {differ} continue from the GPU's tie-band picks", flush=True)
    assert_rel_close(layer.z[:b].cpu(), z, "z")
    assert_rel_close(layer.y_s[:b].cpu(), y_s, "y_s")
    assert_rel_close(y.cpu(), ref, "y")


@pytest.mark.parametrize("b", [1, 2, 4, 5, 8])
def test_moe_block_tiny(k3, b):
    """The fused block entry at the tiny workload against the oracle; dot2
    kernels up to 4 tokens, MFMA above."""
    from moe_router_topk_amd.layer import DecodeLayer
    cfg = synth.MOE_CONFIGS["tiny"]
    w = synth.make_moe_weights(cfg, device=DEV)
    layer = DecodeLayer(w, cfg.k, b_max=8)
    x = synth.make_tokens(cfg, device=DEV, index=80 + b, b=b)
    y = layer.moe_block(x)
    torch.cuda.synchronize()
    assert k3.k3_get_last_dispatch("moe_block") == ("dot2" if b <= 4 else "mfma")
    wc = {key: (v.cpu() if v is not None else None) for key, v in w.items()}
    ref = oracle.moe_block(x.cpu(), wc, cfg.k)
    check_ids(layer.ids[:b], ref["ids"], ref["logits"], cfg.k)
    assert_rel_close(layer.z[:b].cpu(), ref["z"], "z")
    assert_rel_close(layer.y_s[:b].cpu(), ref["y_s"], "y_s")
    assert_rel_close(y.cpu(), ref["y"], "y")


@pytest.mark.parametrize("b,zipf", [(1, 0.0), (2, 0.0), (4, 0.0), (8, 0.0), (16, 0.0),
                                    (40, 0.0), (64, 1.1)])
def test_moe_block_matches_stream_composition(k3, full, b, zipf):
    """k3_moe_block gives the same bits as the separate entry points composed
    on two streams (router+latent, shared expert, routed experts)."""
    from moe_router_topk_amd.layer import DecodeLayer
    cfg, w = full
    w = dict(w)
    w["bias"] = synth.zipf_router_bias(cfg.E, zipf, cfg.seed).to(DEV) if zipf else None
    layer = DecodeLayer(w, cfg.k, b_max=b)
    x = synth.make_tokens(cfg, device=DEV, index=720 + b, b=b)
    y1 = layer.moe_block(x).clone()
    ids1, ys1 = layer.ids[:b].clone(), layer.y_s[:b].clone()
    y2 = layer.moe_block_streams(x)
    torch.cuda.synchronize()
    assert torch.equal(layer.ids[:b], ids1)
    assert torch.equal(layer.y_s[:b], ys1)
    assert torch.equal(y2, y1)


@pytest.mark.parametrize("b,zipf", [(1, 0.0), (4, 0.0), (16, 0.0), (64, 1.1)])
def test_two_stream_combine_waits_for_shared_expert(k3, full, b, zipf):
    """Ordering under stress: the shared expert's side stream starts with a
    spin kernel of fixed, bounded length (it ends on its own) that keeps it
    busy long after the main stream reaches the routed combine, and y_s is
    filled with NaN beforehand. The combine must wait for the side stream's
    event (y_add_ready) before it reads y_s: then y equals the fused block's
    y bit for bit; a combine that read y_s early would see the NaNs."""
    from moe_router_topk_amd.layer import DecodeLayer
    cfg, w = full
    w = dict(w)
    w["bias"] = synth.zipf_router_bias(cfg.E, zipf, cfg.seed).to(DEV) if zipf else None
    layer = DecodeLayer(w, cfg.k, b_max=b)
    m = layer.moe
    x = synth.make_tokens(cfg, device=DEV, index=760 + b, b=b)
    y_ref = layer.moe_block(x).clone()
    ys_ref = layer.y_s[:b].clone()
    torch.cuda.synchronize()
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    ev_in, ev_shared = torch.cuda.Event(), torch.cuda.Event()
    y_s = layer.y_s[:b]
    y_s.fill_(float("nan"))
    y = torch.empty_like(y_ref)
    ev_in.record(main)
    side.wait_event(ev_in)
    with torch.cuda.stream(side):
        # about 8 ms at a 2.4 GHz shader clock: far longer than the main
        # stream's router, latent and routed work before the combine
        torch.cuda._sleep(20_000_000)
    k3.k3_shared_expert(x, m["w13_s"], m["w2_s"], y_s=y_s, workspace=layer.ws_shared,
                        stream=side)
    ev_shared.record(side)
    ids, wts, z = k3.k3_router_topk_latent(x, m["w_router"], m["bias"], cfg.k, m["w_lat"],
                                           workspace=layer.ws_router, stream=main)
    k3.k3_moe_experts(z, ids, wts, m["w13"], m["w2"], y_add=y_s, y_add_ready=ev_shared, y=y,
                      workspace=layer.ws_moe, stream=main)
    torch.cuda.synchronize()
    assert torch.equal(y_s, ys_ref)
    assert torch.isfinite(y.float()).all(), "the combine read y_s before the side stream wrote it"
    assert torch.equal(y, y_ref)


@pytest.mark.parametrize("b", [1, 3, 16])
def test_moe_block_rmsnorm_matches_composition(k3, full, chain_w, b):
    """k3_moe_block_rmsnorm on the o-projection's fp32 h gives the same bits
    as k3_oproj_residual's y_norm fed to k3_moe_block (batch 1 folds the norm
    into the block's first kernel; larger batches run it on its own)."""
    cfg, w = full
    d, K = cfg.d, chain_w["w_o"].shape[1]
    a = synth.randn_bf16((b, K), 1.0, 4, "bn_a", b, device=DEV)
    r = synth.randn_bf16((b, d), 1.0, 4, "bn_r", b, device=DEV)
    g = chain_w["gamma"]
    r1, r2 = r.clone(), r.clone()
    y_norm = k3.k3_oproj_residual(a, chain_w["w_o"], r1, g, 1e-6)
    y1, ids1, wts1, z1, ys1 = k3.k3_moe_block(y_norm, w["w_router"], None, cfg.k, w["w_lat"],
                                              w["w13"], w["w2"], w["w13_s"], w["w2_s"])
    ws = torch.empty(k3.workspace_size("oproj_residual", b=b, K=K, d=d), dtype=torch.uint8,
                     device=DEV)
    assert k3.k3_oproj_residual(a, chain_w["w_o"], r2, None, 1e-6, workspace=ws,
                                norm=False) is None
    h32 = k3.oproj_h32_view(ws, b, d)
    x_out = torch.empty((b, d), dtype=torch.bfloat16, device=DEV)
    y2, ids2, wts2, z2, ys2 = k3.k3_moe_block_rmsnorm(
        h32, g, 1e-6, w["w_router"], None, cfg.k, w["w_lat"], w["w13"], w["w2"], w["w13_s"],
        w["w2_s"], x_out=x_out)
    torch.cuda.synchronize()
    assert torch.equal(r1, r2)
    assert torch.equal(x_out, y_norm)
    assert torch.equal(ids1, ids2) and torch.equal(wts1, wts2) and torch.equal(z1, z2)
    assert torch.equal(ys1, ys2) and torch.equal(y1, y2)
    # without x_out the block keeps x in its workspace
    y3 = k3.k3_moe_block_rmsnorm(h32, g, 1e-6, w["w_router"], None, cfg.k, w["w_lat"], w["w13"],
                                 w["w2"], w["w13_s"], w["w2_s"])[0]
    torch.cuda.synchronize()
    assert torch.equal(y3, y1)


@pytest.mark.parametrize("b,zipf", BLOCK_CASES)
def test_layer_step_chain_then_moe(k3, full, host, chain_w, chain_host, b, zipf):
    """Chain + MoE block, the benchmark's step at each batch it times (b = 1:
    the norm runs in the block's first kernel; above, in the o-projection's
    finishing kernel), against the oracle: the whole chain, then every token
    of the block continued from the bf16 hidden state the GPU produced. The
    side-stream prefetch runs too; it must not change any result."""
    from moe_router_topk_amd.layer import DecodeLayer
    cfg, w = full
    w = dict(w)
    w["bias"] = synth.zipf_router_bias(cfg.E, zipf, cfg.seed).to(DEV) if zipf else None
    layer = DecodeLayer(w, cfg.k, b_max=b, chain=chain_w)
    inp = synth.make_chain_inputs(synth.CHAIN_CONFIG, b, device=DEV)
    r0 = inp["r"].clone()
    y = layer.step(inp["x"], inp["r"], prefetch=True)
    torch.cuda.synchronize()
    c = oracle.chain(inp["x"].cpu(), r0.cpu(), chain_host["w_in"], chain_host["w_o"],
                     chain_host["gamma"], 1e-6)
    assert_rel_close(layer.q[:b].cpu(), c["q"], "q")
    assert_rel_close(inp["r"].cpu(), c["h"], "h")
    assert_rel_close(layer.x_moe[:b].cpu(), c["y"], "x_moe")
    # the MoE block continues from the bf16 hidden state the GPU produced
    bias = w["bias"].cpu() if zipf else None
    ref, z, y_s, _ = _block_reference(layer.x_moe[:b].cpu(), host[0], host[1], bias,
                                      layer.ids[:b], cfg.k, cfg.E)
    assert_rel_close(layer.z[:b].cpu(), z, "z")
    assert_rel_close(y.cpu(), ref, "y")
    # the same step without the prefetch gives the same bits
    inp2 = synth.make_chain_inputs(synth.CHAIN_CONFIG, b, device=DEV)
    y1 = y.clone()
    y2 = layer.step(inp2["x"], inp2["r"], prefetch=False)
    torch.cuda.synchronize()
    assert torch.equal(y2, y1)
