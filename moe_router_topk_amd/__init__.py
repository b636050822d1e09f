"""moe_router_topk_amd -- Python binding of libk3dec (MI355X MoE decode layer).

Every function here marshals torch tensors into the C ABI declared in
include/k3dec.h and raises K3Error on a non-zero status; all arithmetic runs
in the library's HIP kernels. Tensors must live on the GPU; outputs and
workspaces are allocated with torch when the caller does not pass them.
The library is loaded on first use, and loading fails loudly when it has not
been built (python -m moe_router_topk_amd.build).
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "K3Error", "lib", "library_path",
    "k3_router_topk", "k3_router_topk_latent", "k3_proj_skinny", "k3_moe_experts",
    "k3_shared_expert", "k3_oproj_residual", "k3_prefetch", "k3_stream_read", "k3_moe_block",
    "k3_moe_block_rmsnorm", "k3_moe_block_noalloc", "oproj_h32_view",
    "k3_get_last_dispatch", "k3_force_variant",
    "k3_trace_events", "HipEvent",
    "k3_status_string", "k3_version", "workspace_size",
    "OP", "VARIANT", "EXPORTED_SYMBOLS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libk3dec.so")
_lib = None

OP = {"router_topk": 0, "proj_skinny": 1, "moe_experts": 2, "shared_expert": 3,
      "oproj_residual": 4, "prefetch": 5, "router_latent": 6, "moe_block": 7,
      "expert_engine": 8, "dense_pass": 9}
VARIANT = {"none": 0, "dot2": 1, "mfma": 2, "grouped": 3, "stream": 4, "lastwg": 5,
           "wholek": 6, "resident": 7, "splitk": 8}
VARIANT_NAME = {v: k for k, v in VARIANT.items()}

EXPORTED_SYMBOLS = [
    "k3_status_string", "k3_version", "k3_get_last_dispatch", "k3_force_variant",
    "k3_trace_events", "k3_router_topk_workspace_size",
    "k3_router_topk_latent_workspace_size", "k3_proj_skinny_workspace_size",
    "k3_moe_experts_workspace_size", "k3_shared_expert_workspace_size",
    "k3_oproj_residual_workspace_size", "k3_moe_block_workspace_size",
    "k3_moe_block_rmsnorm_workspace_size",
    "k3_router_topk", "k3_router_topk_latent", "k3_proj_skinny", "k3_moe_experts",
    "k3_shared_expert", "k3_oproj_residual", "k3_prefetch", "k3_moe_block",
    "k3_moe_block_rmsnorm", "k3_oproj_residual_h32", "k3_stream_read", "k3_moe_block_noalloc",
]

_vp = ctypes.c_void_p
_i32 = ctypes.c_int
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t


class K3Error(RuntimeError):
    """A libk3dec entry point returned a non-zero status."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {k3_status_string(status)}")


def library_path() -> str:
    return _LIB_PATH


def lib():
    """The loaded libk3dec (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"libk3dec is not built ({_LIB_PATH} missing); run "
            "`python -m moe_router_topk_amd.build` first. There is no fallback path.")
    L = ctypes.CDLL(_LIB_PATH)
    L.k3_status_string.restype = ctypes.c_char_p
    L.k3_status_string.argtypes = [_i32]
    L.k3_version.restype = _i32
    L.k3_get_last_dispatch.argtypes = [_i32]
    L.k3_get_last_dispatch.restype = _i32
    L.k3_force_variant.argtypes = [_i32, _i32]
    L.k3_force_variant.restype = _i32
    L.k3_trace_events.argtypes = [_i32, _vp, _vp]
    L.k3_trace_events.restype = _i32
    L.k3_router_topk_workspace_size.argtypes = [_i32, _i32]
    L.k3_router_topk_latent_workspace_size.argtypes = [_i32, _i32, _i32]
    L.k3_proj_skinny_workspace_size.argtypes = [_i32, _i32, _i32]
    L.k3_moe_experts_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32]
    L.k3_shared_expert_workspace_size.argtypes = [_i32, _i32, _i32]
    L.k3_oproj_residual_workspace_size.argtypes = [_i32, _i32, _i32]
    L.k3_moe_block_workspace_size.argtypes = [_i32] * 7
    L.k3_moe_block_rmsnorm_workspace_size.argtypes = [_i32] * 7
    for f in ("k3_router_topk_workspace_size", "k3_router_topk_latent_workspace_size",
              "k3_proj_skinny_workspace_size",
              "k3_moe_experts_workspace_size", "k3_shared_expert_workspace_size",
              "k3_oproj_residual_workspace_size", "k3_moe_block_workspace_size",
              "k3_moe_block_rmsnorm_workspace_size"):
        getattr(L, f).restype = _sz
    L.k3_moe_block_rmsnorm.argtypes = [_vp, _i32, _i32, _vp, ctypes.c_float, _vp, _vp, _vp, _i32,
                                       _i32, _vp, _i32, _vp, _vp, _i32, _vp, _vp, _i32, _vp, _vp,
                                       _vp, _i64, _vp, _vp, _vp, _sz, _vp]
    L.k3_moe_block_rmsnorm.restype = _i32
    L.k3_oproj_residual_h32.argtypes = [_vp]
    L.k3_oproj_residual_h32.restype = _vp
    L.k3_moe_block.argtypes = [_vp, _i64, _i32, _i32, _vp, _vp, _i32, _i32, _vp, _i32, _vp, _vp,
                               _i32, _vp, _vp, _i32, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _sz, _vp]
    L.k3_moe_block.restype = _i32
    L.k3_moe_block_noalloc.argtypes = [_vp, _i64, _i32, _i32, _vp, _vp, _i32, _i32, _vp, _i32,
                                       _vp, _vp, _i32, _vp, _vp, _i32, _vp, _vp, _vp, _i64, _vp,
                                       _vp, _vp]
    L.k3_moe_block_noalloc.restype = _i32
    L.k3_router_topk.argtypes = [_vp, _i64, _i32, _i32, _vp, _vp, _i32, _i32, _vp, _vp, _vp,
                                 _sz, _vp]
    L.k3_router_topk_latent.argtypes = [_vp, _i64, _i32, _i32, _vp, _vp, _i32, _i32, _vp, _i32,
                                        _vp, _vp, _vp, _i64, _vp, _sz, _vp]
    L.k3_proj_skinny.argtypes = [_vp, _i64, _i32, _i32, _vp, _i32, _vp, _i64, _vp, _sz, _vp]
    L.k3_moe_experts.argtypes = [_vp, _i64, _i32, _i32, _vp, _vp, _i32, _vp, _vp, _i32, _i32,
                                 _i32, _vp, _vp, _vp, _i32, _vp, _sz, _vp]
    L.k3_shared_expert.argtypes = [_vp, _i64, _i32, _i32, _vp, _vp, _i32, _vp, _i32, _vp, _sz,
                                   _vp]
    L.k3_oproj_residual.argtypes = [_vp, _i64, _i32, _i32, _vp, _i32, _vp, _vp, ctypes.c_float,
                                    _vp, _vp, _sz, _vp]
    L.k3_prefetch.argtypes = [_vp, _sz, _i32, _vp]
    L.k3_stream_read.argtypes = [_vp, _sz, _vp]
    for f in ("k3_router_topk", "k3_router_topk_latent", "k3_proj_skinny", "k3_moe_experts",
              "k3_shared_expert", "k3_oproj_residual", "k3_prefetch", "k3_stream_read"):
        getattr(L, f).restype = _i32
    _lib = L
    return _lib


def k3_status_string(status: int) -> str:
    return lib().k3_status_string(int(status)).decode()


def k3_version() -> int:
    return lib().k3_version()


def k3_get_last_dispatch(op) -> str:
    return VARIANT_NAME.get(lib().k3_get_last_dispatch(OP[op] if isinstance(op, str) else op),
                            "unknown")


def k3_force_variant(op, variant) -> None:
    o = OP[op] if isinstance(op, str) else op
    v = VARIANT[variant] if isinstance(variant, str) else variant
    _check("k3_force_variant", lib().k3_force_variant(o, v))


_hip = None


def _hiprt():
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        _hip.hipEventDestroy.argtypes = [_vp]
        _hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), _vp, _vp]
        _hip.hipGetLastError.restype = ctypes.c_int
    return _hip


class HipEvent:
    """A raw hipEvent_t with timing enabled, for k3_trace_events (torch only
    times events it recorded itself)."""

    def __init__(self):
        self.handle = ctypes.c_void_p()
        rc = _hiprt().hipEventCreate(ctypes.byref(self.handle))
        if rc != 0:
            _hiprt().hipGetLastError()
            raise RuntimeError(f"hipEventCreate failed ({rc})")

    def elapsed_ms(self, end: "HipEvent") -> float:
        ms = ctypes.c_float()
        rc = _hiprt().hipEventElapsedTime(ctypes.byref(ms), self.handle, end.handle)
        if rc != 0:
            _hiprt().hipGetLastError()  # clear it, or the next runtime call reports it
            raise RuntimeError(f"hipEventElapsedTime failed ({rc}): event not recorded?")
        return ms.value

    def __del__(self):
        if _hip is not None and self.handle:
            _hip.hipEventDestroy(self.handle)
            self.handle = ctypes.c_void_p()


def k3_trace_events(op, begin, end) -> None:
    """Record the HipEvent pair (begin, end) around the main kernel of every
    following call of `op`; (None, None) clears."""
    o = OP[op] if isinstance(op, str) else op
    b = None if begin is None else begin.handle
    e = None if end is None else end.handle
    _check("k3_trace_events", lib().k3_trace_events(o, b, e))


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise K3Error(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _ld(t) -> int:
    assert t.dim() == 2 and t.stride(1) == 1, "rows must be contiguous"
    return t.stride(0)


def _dev(t):
    if not t.is_cuda:
        raise ValueError("libk3dec works on GPU tensors only")
    return t.device


_ws_cache: dict = {}


def _workspace(device, nbytes: int, tag: str):
    """A cached scratch buffer of at least nbytes on device, one per entry
    point, so calls of different entry points on different streams never
    share scratch. Two in-flight calls of the same entry point must pass
    their own workspaces."""
    if nbytes == 0:
        return None
    key = (device.index if device.index is not None else torch.cuda.current_device(), tag)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        # zeroed once: the forced last-workgroup router keeps its counter in
        # the workspace head, which must start at zero (and stays zero)
        buf = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf


def workspace_size(op: str, **kw) -> int:
    L = lib()
    if op == "router_topk":
        return L.k3_router_topk_workspace_size(kw["b"], kw["E"])
    if op == "router_topk_latent":
        return L.k3_router_topk_latent_workspace_size(kw["b"], kw["E"], kw["d_lat"])
    if op == "proj_skinny":
        return L.k3_proj_skinny_workspace_size(kw["b"], kw["K"], kw["N"])
    if op == "moe_experts":
        return L.k3_moe_experts_workspace_size(kw["b"], kw["d_in"], kw["E"], kw["k"], kw["I"],
                                               kw["d_out"])
    if op == "shared_expert":
        return L.k3_shared_expert_workspace_size(kw["b"], kw["d"], kw["I"])
    if op == "oproj_residual":
        return L.k3_oproj_residual_workspace_size(kw["b"], kw["K"], kw["d"])
    if op == "moe_block_rmsnorm":
        return L.k3_moe_block_rmsnorm_workspace_size(kw["b"], kw["d"], kw["E"], kw["k"],
                                                     kw["d_lat"], kw["I"], kw["I_s"])
    if op == "moe_block":
        return L.k3_moe_block_workspace_size(kw["b"], kw["d"], kw["E"], kw["k"], kw["d_lat"],
                                             kw["I"], kw["I_s"])
    raise ValueError(op)


# ------------------------------------------------------------------ entry points
def k3_router_topk(x, w_router, bias, k, topk_ids=None, topk_w=None, workspace=None,
                   stream=None):
    """(topk_ids [b x k] int32, topk_w [b x k] fp32) for x [b x d] bf16. A caller's
    workspace must start with 4 zero bytes for the forced "lastwg" variant."""
    dev = _dev(x)
    b, d = x.shape
    E = w_router.shape[0]
    if topk_ids is None:
        topk_ids = torch.empty((b, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((b, k), dtype=torch.float32, device=dev)
    nbytes = lib().k3_router_topk_workspace_size(b, E)
    ws = workspace if workspace is not None else _workspace(dev, nbytes, "router_topk")
    _check("k3_router_topk", lib().k3_router_topk(
        _ptr(x), _ld(x), b, d, _ptr(w_router), _ptr(bias), E, k, _ptr(topk_ids), _ptr(topk_w),
        _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)))
    return topk_ids, topk_w


def k3_router_topk_latent(x, w_router, bias, k, w_lat, topk_ids=None, topk_w=None, z=None,
                          workspace=None, stream=None):
    """(topk_ids, topk_w, z): router top-k and the latent projection z = x . w_lat^T
    from one pass over x."""
    dev = _dev(x)
    b, d = x.shape
    E = w_router.shape[0]
    d_lat = w_lat.shape[0]
    if topk_ids is None:
        topk_ids = torch.empty((b, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((b, k), dtype=torch.float32, device=dev)
    if z is None:
        z = torch.empty((b, d_lat), dtype=torch.bfloat16, device=dev)
    nbytes = lib().k3_router_topk_latent_workspace_size(b, E, d_lat)
    ws = workspace if workspace is not None else _workspace(dev, nbytes, "router_topk_latent")
    _check("k3_router_topk_latent", lib().k3_router_topk_latent(
        _ptr(x), _ld(x), b, d, _ptr(w_router), _ptr(bias), E, k, _ptr(w_lat), d_lat,
        _ptr(topk_ids), _ptr(topk_w), _ptr(z), _ld(z), _ptr(ws),
        ws.numel() if ws is not None else 0, _stream(stream)))
    return topk_ids, topk_w, z


def k3_proj_skinny(x, w, y=None, workspace=None, stream=None):
    """y [b x N] bf16 = x [b x K] . w[N x K]^T."""
    dev = _dev(x)
    b, K = x.shape
    N = w.shape[0]
    if y is None:
        y = torch.empty((b, N), dtype=torch.bfloat16, device=dev)
    nbytes = lib().k3_proj_skinny_workspace_size(b, K, N)
    ws = workspace if workspace is not None else _workspace(dev, nbytes, "proj_skinny")
    _check("k3_proj_skinny", lib().k3_proj_skinny(
        _ptr(x), _ld(x), b, K, _ptr(w), N, _ptr(y), _ld(y), _ptr(ws),
        ws.numel() if ws is not None else 0, _stream(stream)))
    return y


def k3_moe_experts(z, topk_ids, topk_w, w13, w2, y_add=None, y_add_ready=None, y=None,
                   cu_budget=0, workspace=None, stream=None):
    """y [b x d_out] bf16 = y_add + sum_j w_j Expert_{ids_j}(z)."""
    dev = _dev(z)
    b, d_in = z.shape
    k = topk_ids.shape[1]
    E, twoI, _ = w13.shape
    I = twoI // 2
    d_out = w2.shape[1]
    if y is None:
        y = torch.empty((b, d_out), dtype=torch.bfloat16, device=dev)
    nbytes = lib().k3_moe_experts_workspace_size(b, d_in, E, k, I, d_out)
    ws = workspace if workspace is not None else _workspace(dev, nbytes, "moe_experts")
    ev = None
    if y_add_ready is not None:
        ev = ctypes.c_void_p(y_add_ready.cuda_event if hasattr(y_add_ready, "cuda_event")
                             else int(y_add_ready))
    _check("k3_moe_experts", lib().k3_moe_experts(
        _ptr(z), _ld(z), b, d_in, _ptr(topk_ids), _ptr(topk_w), k, _ptr(w13), _ptr(w2), E, I,
        d_out, _ptr(y_add), ev, _ptr(y), int(cu_budget), _ptr(ws),
        ws.numel() if ws is not None else 0, _stream(stream)))
    return y


def k3_shared_expert(x, w13, w2, y_s=None, cu_budget=0, workspace=None, stream=None):
    """y_s [b x d] fp32 = shared SwiGLU expert of x [b x d] bf16."""
    dev = _dev(x)
    b, d = x.shape
    I = w13.shape[0] // 2
    if y_s is None:
        y_s = torch.empty((b, d), dtype=torch.float32, device=dev)
    nbytes = lib().k3_shared_expert_workspace_size(b, d, I)
    ws = workspace if workspace is not None else _workspace(dev, nbytes, "shared_expert")
    _check("k3_shared_expert", lib().k3_shared_expert(
        _ptr(x), _ld(x), b, d, _ptr(w13), _ptr(w2), I, _ptr(y_s), int(cu_budget), _ptr(ws),
        ws.numel() if ws is not None else 0, _stream(stream)))
    return y_s


def k3_oproj_residual(a, w_o, residual, gamma, eps, y_norm=None, workspace=None, stream=None,
                      norm=True):
    """In place: residual <- bf16(residual + a . w_o^T); returns y_norm = RMSNorm(h) * gamma.
    With norm=False the norm is skipped (returns None); the fp32 h stays in the workspace
    (oproj_h32_view)."""
    dev = _dev(a)
    b, K = a.shape
    d = w_o.shape[0]
    assert residual.is_contiguous() and residual.shape == (b, d)
    if y_norm is None and norm:
        y_norm = torch.empty((b, d), dtype=torch.bfloat16, device=dev)
    nbytes = lib().k3_oproj_residual_workspace_size(b, K, d)
    ws = workspace if workspace is not None else _workspace(dev, nbytes, "oproj_residual")
    _check("k3_oproj_residual", lib().k3_oproj_residual(
        _ptr(a), _ld(a), b, K, _ptr(w_o), d, _ptr(residual), _ptr(gamma), float(eps),
        _ptr(y_norm), _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)))
    return y_norm


def k3_moe_block(x, w_router, bias, k, w_lat, w13, w2, w13_s, w2_s, topk_ids=None,
                 topk_w=None, z=None, y_s=None, y=None, workspace=None, stream=None):
    """The whole MoE block on one stream: returns (y, topk_ids, topk_w, z, y_s)."""
    dev = _dev(x)
    b, d = x.shape
    E = w_router.shape[0]
    d_lat = w_lat.shape[0]
    I = w13.shape[1] // 2
    I_s = w13_s.shape[0] // 2
    if topk_ids is None:
        topk_ids = torch.empty((b, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((b, k), dtype=torch.float32, device=dev)
    if z is None:
        z = torch.empty((b, d_lat), dtype=torch.bfloat16, device=dev)
    if y_s is None:
        y_s = torch.empty((b, d), dtype=torch.float32, device=dev)
    if y is None:
        y = torch.empty((b, d), dtype=torch.bfloat16, device=dev)
    nbytes = lib().k3_moe_block_workspace_size(b, d, E, k, d_lat, I, I_s)
    ws = workspace if workspace is not None else _workspace(dev, nbytes, "moe_block")
    _check("k3_moe_block", lib().k3_moe_block(
        _ptr(x), _ld(x), b, d, _ptr(w_router), _ptr(bias), E, k, _ptr(w_lat), d_lat, _ptr(w13),
        _ptr(w2), I, _ptr(w13_s), _ptr(w2_s), I_s, _ptr(topk_ids), _ptr(topk_w), _ptr(z), _ld(z),
        _ptr(y_s), _ptr(y), _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)))
    return y, topk_ids, topk_w, z, y_s


def k3_moe_block_noalloc(x, w_router, bias, k, w_lat, w13, w2, w13_s, w2_s, topk_ids=None,
                         topk_w=None, z=None, y_s=None, y=None, stream=None):
    """k3_moe_block with the library's static scratch instead of a workspace
    (the library allocates nothing; outputs are allocated here when not
    passed): returns (y, topk_ids, topk_w, z, y_s)."""
    dev = _dev(x)
    b, d = x.shape
    E = w_router.shape[0]
    d_lat = w_lat.shape[0]
    I = w13.shape[1] // 2
    I_s = w13_s.shape[0] // 2
    if topk_ids is None:
        topk_ids = torch.empty((b, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((b, k), dtype=torch.float32, device=dev)
    if z is None:
        z = torch.empty((b, d_lat), dtype=torch.bfloat16, device=dev)
    if y_s is None:
        y_s = torch.empty((b, d), dtype=torch.float32, device=dev)
    if y is None:
        y = torch.empty((b, d), dtype=torch.bfloat16, device=dev)
    _check("k3_moe_block_noalloc", lib().k3_moe_block_noalloc(
        _ptr(x), _ld(x), b, d, _ptr(w_router), _ptr(bias), E, k, _ptr(w_lat), d_lat, _ptr(w13),
        _ptr(w2), I, _ptr(w13_s), _ptr(w2_s), I_s, _ptr(topk_ids), _ptr(topk_w), _ptr(z), _ld(z),
        _ptr(y_s), _ptr(y), _stream(stream)))
    return y, topk_ids, topk_w, z, y_s


def oproj_h32_view(workspace, b, d):
    """The fp32 h [b x d] that k3_oproj_residual left in `workspace` (a view, no copy)."""
    off = lib().k3_oproj_residual_h32(_ptr(workspace)) - workspace.data_ptr()
    return workspace[off:off + 4 * b * d].view(torch.float32).view(b, d)


def k3_moe_block_rmsnorm(h32, gamma, eps, w_router, bias, k, w_lat, w13, w2, w13_s, w2_s,
                         x_out=None, topk_ids=None, topk_w=None, z=None, y_s=None, y=None,
                         workspace=None, stream=None):
    """The MoE block on x = RMSNorm(h32) * gamma (normalised inside the block):
    returns (y, topk_ids, topk_w, z, y_s); x_out, if given, receives x."""
    dev = _dev(h32)
    b, d = h32.shape
    assert h32.dtype == torch.float32 and h32.is_contiguous()
    E = w_router.shape[0]
    d_lat = w_lat.shape[0]
    I = w13.shape[1] // 2
    I_s = w13_s.shape[0] // 2
    if topk_ids is None:
        topk_ids = torch.empty((b, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((b, k), dtype=torch.float32, device=dev)
    if z is None:
        z = torch.empty((b, d_lat), dtype=torch.bfloat16, device=dev)
    if y_s is None:
        y_s = torch.empty((b, d), dtype=torch.float32, device=dev)
    if y is None:
        y = torch.empty((b, d), dtype=torch.bfloat16, device=dev)
    nbytes = lib().k3_moe_block_rmsnorm_workspace_size(b, d, E, k, d_lat, I, I_s)
    ws = workspace if workspace is not None else _workspace(dev, nbytes, "moe_block_rmsnorm")
    _check("k3_moe_block_rmsnorm", lib().k3_moe_block_rmsnorm(
        _ptr(h32), b, d, _ptr(gamma), float(eps), _ptr(x_out), _ptr(w_router), _ptr(bias), E, k,
        _ptr(w_lat), d_lat, _ptr(w13), _ptr(w2), I, _ptr(w13_s), _ptr(w2_s), I_s,
        _ptr(topk_ids), _ptr(topk_w), _ptr(z), _ld(z), _ptr(y_s), _ptr(y), _ptr(ws),
        ws.numel() if ws is not None else 0, _stream(stream)))
    return y, topk_ids, topk_w, z, y_s


def k3_prefetch(t, nbytes=None, cu_budget=0, stream=None):
    """Read the first nbytes of tensor t (default: all of it) into the MALL."""
    nbytes = t.numel() * t.element_size() if nbytes is None else int(nbytes)
    _check("k3_prefetch", lib().k3_prefetch(_ptr(t), nbytes, int(cu_budget), _stream(stream)))


def k3_stream_read(t, nbytes=None, stream=None):
    """Read the first nbytes of tensor t (default: all of it) with the weight
    streams' non-temporal loads and discard them (streaming-read ceiling)."""
    nbytes = t.numel() * t.element_size() if nbytes is None else int(nbytes)
    _check("k3_stream_read", lib().k3_stream_read(_ptr(t), nbytes, _stream(stream)))
