"""One decode layer step on one GPU: stream and event orchestration only.

"Hyper Optimizing Kimi K3 in vLLM", Part 1:
  section 1 -- attention input projection (k3_proj_skinny);
  section 2 -- output projection fused with the attention residual
               (k3_oproj_residual; the RMSNorm that feeds the MoE runs in the
               block's first kernel, k3_moe_block_rmsnorm);
  section 3 -- router scores and latent projection from the same input, then
               the routed experts; the shared expert on a separate stream,
               overlapping routing and the routed experts, with a bounded
               share of the GPU (cu_budget);
  section 4 -- a side-stream prefetch of upcoming weights.

The attention core is not part of this library: the output projection reads
the first K_o columns of the input projection's output in its place.

All buffers are allocated once, at construction; a step launches kernels only
(no allocation, no host synchronisation), so it can be captured in a graph.
"""
from __future__ import annotations

import torch

from . import (k3_moe_block, k3_moe_block_rmsnorm, k3_moe_experts, k3_oproj_residual,
               k3_prefetch, k3_proj_skinny, k3_router_topk_latent, k3_shared_expert,
               oproj_h32_view, workspace_size)


class DecodeLayer:
    """Weights of one layer plus the scratch a step needs at batch <= b_max.

    moe: w_router [E x d], bias ([E] fp32 or None), w_lat [d_lat x d],
         w13 [E x 2I x d_lat], w2 [E x d x I], w13_s [2I_s x d], w2_s [d x I_s]
    chain (optional): w_in [N_in x d], w_o [d x K_o], gamma [d]
    """

    def __init__(self, moe: dict, k: int, b_max: int = 64, chain: dict | None = None,
                 eps: float = 1e-6, cu_shared: int = 0, prefetch_cu: int = 0):
        self.moe = moe
        self.chain_w = chain
        self.k = k
        self.eps = eps
        self.cu_shared = cu_shared
        self.prefetch_cu = prefetch_cu
        dev = moe["w_router"].device
        self.device = dev
        E, d = moe["w_router"].shape
        d_lat = moe["w_lat"].shape[0]
        I = moe["w13"].shape[1] // 2
        I_s = moe["w13_s"].shape[0] // 2
        self.E, self.d, self.d_lat, self.I, self.I_s, self.b_max = E, d, d_lat, I, I_s, b_max
        u8 = dict(dtype=torch.uint8, device=dev)
        self.ws_router = torch.empty(
            workspace_size("router_topk_latent", b=b_max, E=E, d_lat=d_lat), **u8)
        self.ws_moe = torch.empty(
            workspace_size("moe_experts", b=b_max, d_in=d_lat, E=E, k=k, I=I, d_out=d), **u8)
        self.ws_shared = torch.empty(workspace_size("shared_expert", b=b_max, d=d, I=I_s), **u8)
        # sized for the block that normalises its own input (the larger one)
        self.ws_block = torch.empty(workspace_size("moe_block_rmsnorm", b=b_max, d=d, E=E, k=k,
                                                   d_lat=d_lat, I=I, I_s=I_s), **u8)
        self.ids = torch.empty((b_max, k), dtype=torch.int32, device=dev)
        self.wts = torch.empty((b_max, k), dtype=torch.float32, device=dev)
        self.z = torch.empty((b_max, d_lat), dtype=torch.bfloat16, device=dev)
        self.y_s = torch.empty((b_max, d), dtype=torch.float32, device=dev)
        self.y = torch.empty((b_max, d), dtype=torch.bfloat16, device=dev)
        if chain is not None:
            n_in = chain["w_in"].shape[0]
            self.k_o = chain["w_o"].shape[1]
            self.q = torch.empty((b_max, n_in), dtype=torch.bfloat16, device=dev)
            self.x_moe = torch.empty((b_max, d), dtype=torch.bfloat16, device=dev)
            self.ws_oproj = torch.empty(
                workspace_size("oproj_residual", b=b_max, K=self.k_o, d=d), **u8)
            self.ws_proj = torch.empty(
                workspace_size("proj_skinny", b=b_max, K=d, N=n_in), **u8)
        self.side = torch.cuda.Stream(device=dev)
        self.pf_stream = torch.cuda.Stream(device=dev)
        self.ev_in = torch.cuda.Event()
        self.ev_shared = torch.cuda.Event()
        self.ev_side_done = torch.cuda.Event()

    # -------------------------------------------------------------- MoE block
    def moe_block(self, x: torch.Tensor) -> torch.Tensor:
        """y [b x d] bf16 = shared(x) + sum_j w_j routed_j(latent(x)), one
        stream (k3_moe_block)."""
        b = x.shape[0]
        assert b <= self.b_max
        m = self.moe
        y, _, _, _, _ = k3_moe_block(
            x, m["w_router"], m["bias"], self.k, m["w_lat"], m["w13"], m["w2"], m["w13_s"],
            m["w2_s"], topk_ids=self.ids[:b], topk_w=self.wts[:b], z=self.z[:b],
            y_s=self.y_s[:b], y=self.y[:b], workspace=self.ws_block)
        return y

    def moe_block_streams(self, x: torch.Tensor) -> torch.Tensor:
        """The same block composed from the separate entry points, with the
        shared expert on a second stream (joined before the combine)."""
        b = x.shape[0]
        assert b <= self.b_max
        m = self.moe
        main = torch.cuda.current_stream(self.device)
        self.ev_in.record(main)
        self.side.wait_event(self.ev_in)
        y_s = self.y_s[:b]
        k3_shared_expert(x, m["w13_s"], m["w2_s"], y_s=y_s, cu_budget=self.cu_shared,
                         workspace=self.ws_shared, stream=self.side)
        self.ev_shared.record(self.side)
        ids, wts, z = self.ids[:b], self.wts[:b], self.z[:b]
        k3_router_topk_latent(x, m["w_router"], m["bias"], self.k, m["w_lat"], topk_ids=ids,
                              topk_w=wts, z=z, workspace=self.ws_router, stream=main)
        y = self.y[:b]
        k3_moe_experts(z, ids, wts, m["w13"], m["w2"], y_add=y_s, y_add_ready=self.ev_shared,
                       y=y, workspace=self.ws_moe, stream=main)
        return y

    # -------------------------------------------------------------- chain
    def attn_chain(self, x: torch.Tensor, residual: torch.Tensor) -> torch.Tensor:
        """q = x . W_in^T; residual <- residual + q[:, :K_o] . W_o^T (in place);
        returns RMSNorm(residual) * gamma."""
        c = self.chain_w
        b = x.shape[0]
        q = self.q[:b]
        k3_proj_skinny(x, c["w_in"], y=q, workspace=self.ws_proj)
        x_moe = self.x_moe[:b]
        k3_oproj_residual(q[:, :self.k_o], c["w_o"], residual, c["gamma"], self.eps,
                          y_norm=x_moe, workspace=self.ws_oproj)
        return x_moe

    def attn_chain_h32(self, x: torch.Tensor, residual: torch.Tensor) -> torch.Tensor:
        """As attn_chain without the norm: returns the fp32 h (a view into the
        o-projection's workspace) for moe_block_rmsnorm."""
        c = self.chain_w
        b = x.shape[0]
        q = self.q[:b]
        k3_proj_skinny(x, c["w_in"], y=q, workspace=self.ws_proj)
        k3_oproj_residual(q[:, :self.k_o], c["w_o"], residual, None, self.eps,
                          workspace=self.ws_oproj, norm=False)
        return oproj_h32_view(self.ws_oproj, b, self.d)

    def moe_block_rmsnorm(self, h32: torch.Tensor) -> torch.Tensor:
        """The MoE block on RMSNorm(h32) * gamma, normalised inside the block
        (k3_moe_block_rmsnorm); the normalised input lands in x_moe."""
        b = h32.shape[0]
        assert b <= self.b_max
        m = self.moe
        y, _, _, _, _ = k3_moe_block_rmsnorm(
            h32, self.chain_w["gamma"], self.eps, m["w_router"], m["bias"], self.k, m["w_lat"],
            m["w13"], m["w2"], m["w13_s"], m["w2_s"], x_out=self.x_moe[:b],
            topk_ids=self.ids[:b], topk_w=self.wts[:b], z=self.z[:b], y_s=self.y_s[:b],
            y=self.y[:b], workspace=self.ws_block)
        return y

    PREFETCH_KEYS = ("w_router", "w_lat")

    def step(self, x: torch.Tensor, residual: torch.Tensor, prefetch: bool = False):
        """The whole hot path of a decode layer: chain, then the MoE block on
        the normalised hidden state. With prefetch, a side stream reads the
        router and latent weights (the MoE block's first reads) into the MALL
        while the chain runs, on prefetch_cu compute units; the main stream
        joins it only at the end of the step."""
        main = torch.cuda.current_stream(self.device)
        if prefetch:
            self.ev_in.record(main)
            self.pf_stream.wait_event(self.ev_in)
            for key in self.PREFETCH_KEYS:
                k3_prefetch(self.moe[key], cu_budget=self.prefetch_cu, stream=self.pf_stream)
            self.ev_side_done.record(self.pf_stream)
        # one token: the chain leaves the fp32 h and the block normalises it in
        # its first kernel; more tokens: the o-projection's finishing kernel
        # normalises (each saves a kernel boundary)
        if x.shape[0] == 1:
            y = self.moe_block_rmsnorm(self.attn_chain_h32(x, residual))
        else:
            y = self.moe_block(self.attn_chain(x, residual))
        if prefetch:
            main.wait_event(self.ev_side_done)
        return y
