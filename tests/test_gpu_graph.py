"""The decode-layer step captured in a HIP graph (as the benchmark times it):
every replay must give the eager result bit for bit, with eager work and
synchronisation between replays, and trace events recorded inside the
graph must time the traced kernel."""
import math

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def k3():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need one")
    import moe_router_topk_amd as k3
    k3.lib()
    return k3


def _tiny_layer(prefetch_cu=8):
    from moe_router_topk_amd.layer import DecodeLayer
    cfg = synth.MOE_CONFIGS["tiny"]
    w = synth.make_moe_weights(cfg, device=DEV)
    chain = {
        "w_in": synth.randn_bf16((384, 256), 1 / math.sqrt(256), 3, "g_w_in", device=DEV),
        "w_o": synth.randn_bf16((256, 256), 1 / math.sqrt(256), 3, "g_w_o", device=DEV),
        "gamma": torch.ones(256, dtype=torch.bfloat16, device=DEV),
    }
    return DecodeLayer(w, cfg.k, b_max=64, chain=chain, prefetch_cu=prefetch_cu)


@pytest.mark.parametrize("b", [1, 4, 8, 64])
def test_step_graph_replays_match_eager(k3, b):
    layer = _tiny_layer()
    x = synth.randn_bf16((b, 256), 1.0, 5, "g_x", b, device=DEV)
    r = synth.randn_bf16((b, 256), 1.0, 5, "g_r", b, device=DEV)
    r_e = r.clone()
    y_e = layer.step(x, r_e, prefetch=True).clone()
    ids_e = layer.ids[:b].clone()
    torch.cuda.synchronize()

    r_g = r.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        y_g = layer.step(x, r_g, prefetch=True)
    other_x = synth.randn_bf16((b, 256), 1.0, 6, "g_x2", b, device=DEV)
    for rep in range(4):
        r_g.copy_(r)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_g, y_e), f"replay {rep}: y differs from eager"
        assert torch.equal(r_g, r_e), f"replay {rep}: residual differs from eager"
        assert torch.equal(layer.ids[:b], ids_e)
        # eager work on the same buffers between replays
        layer.moe_block(other_x)
        torch.cuda.synchronize()


def test_trace_events_time_eager_calls(k3):
    """The trace hook brackets the routed gate/up kernel of an eager call."""
    layer = _tiny_layer()
    x = synth.randn_bf16((1, 256), 1.0, 7, "t_x", device=DEV)
    kb, ke = k3.HipEvent(), k3.HipEvent()
    layer.moe_block(x)
    torch.cuda.synchronize()
    k3.k3_trace_events("moe_experts", kb, ke)
    try:
        layer.moe_block(x)
    finally:
        k3.k3_trace_events("moe_experts", None, None)
    torch.cuda.synchronize()
    ms = kb.elapsed_ms(ke)
    assert 0.0 < ms < 50.0, ms


def test_trace_hook_is_harmless_in_capture(k3):
    """Inside a capture the trace records are only dependency marks: the call
    still succeeds and the replay still matches eager."""
    layer = _tiny_layer()
    x = synth.randn_bf16((1, 256), 1.0, 8, "t_x2", device=DEV)
    y_e = layer.moe_block(x).clone()
    torch.cuda.synchronize()
    kb, ke = k3.HipEvent(), k3.HipEvent()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        k3.k3_trace_events("moe_experts", kb, ke)
        y = layer.moe_block(x)
    k3.k3_trace_events("moe_experts", None, None)
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(y, y_e)
