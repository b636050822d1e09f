"""k3_moe_block_noalloc (the MoE block on the library's static scratch, for
callers that cannot allocate) against k3_moe_block with a workspace: two
calls in a row on the full-size layer, the second with a smaller batch, each
bit for bit the same as the workspace entry point on the same inputs."""
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


def test_noalloc_matches_workspace_entry(k3):
    cfg = synth.MOE_CONFIGS["b1"]
    w = synth.make_moe_weights(cfg, device=DEV)
    torch.cuda.synchronize()
    # the larger call first (64 tokens, Zipf router bias: 27.7 MiB of the
    # 32 MiB scratch), then a smaller one (16 tokens, uniform routing) that
    # finds the first call's contents in the scratch
    for b, zipf in ((64, 1.1), (16, 0.0)):
        print(f"no-alloc block b={b} zipf={zipf}", flush=True)
        bias = synth.zipf_router_bias(cfg.E, zipf, cfg.seed).to(DEV) if zipf else None
        x = synth.make_tokens(cfg, device=DEV, index=800 + b, b=b)
        args = (x, w["w_router"], bias, cfg.k, w["w_lat"], w["w13"], w["w2"], w["w13_s"],
                w["w2_s"])
        ref = [t.clone() for t in k3.k3_moe_block(*args)]
        torch.cuda.synchronize()
        got = k3.k3_moe_block_noalloc(*args)
        torch.cuda.synchronize()
        for name, a, r in zip(("y", "topk_ids", "topk_w", "z", "y_s"), got, ref):
            assert torch.equal(a, r), f"b={b}: {name} differs from k3_moe_block"
        assert k3.k3_get_last_dispatch("moe_block") == "mfma"


def test_noalloc_rejects_oversized_shape(k3):
    """A shape that needs more than the static scratch fails with
    K3_ERR_SCRATCH and launches nothing."""
    E, d, I, k, b = 1024, 8192, 8192, 32, 64
    x = torch.zeros((b, d), dtype=torch.bfloat16, device=DEV)
    small = torch.zeros((16,), dtype=torch.bfloat16, device=DEV)
    L = k3.lib()
    out = torch.zeros((b * max(k, d),), dtype=torch.float32, device=DEV)
    p = out.data_ptr()
    st = L.k3_moe_block_noalloc(x.data_ptr(), d, b, d, small.data_ptr(), None, E, k,
                                small.data_ptr(), d, small.data_ptr(), small.data_ptr(), I,
                                small.data_ptr(), small.data_ptr(), I, p, p, p, d, p, p, None)
    torch.cuda.synchronize()
    assert st == -5
    assert (out == 0).all()
