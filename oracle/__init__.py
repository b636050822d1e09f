"""The oracle: plain fp64 CPU implementation of the MoE decode layer.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this package. The GPU library never
imports, links or calls it, and the two share no code; the only module both
sides use is the seeded input generator (``synth``), which holds no part of
the layer's arithmetic.

The arithmetic lives in ``k3_oracle.c`` (plain C, gcc -O2, no fast-math,
OpenMP over independent outputs only); this wrapper only marshals arrays and
composes the steps in the order "Hyper Optimizing Kimi K3 in vLLM: Moving
Fast and Responsibly" gives them (Part 1, section 3: router and latent from
the same input, then the routed experts, with the shared expert beside them;
Part 1, sections 1-2: input projection, then output projection with the
attention residual). bf16 inputs are widened exactly; every intermediate
stays in fp64 unless a caller passes the bf16 tensors a GPU call received.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(closed forms, invariants, brute force on tiny inputs and hand-derived
values); none is "parity unpinned".
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "k3_oracle.c")
_LIB = os.path.join(_HERE, "libk3oracle.so")
_lib = None

_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_i64 = ctypes.c_int64
_int = ctypes.c_int


def build(force: bool = True) -> str:
    """Compile k3_oracle.c into libk3oracle.so with gcc (plain -O2, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-Wall", "-shared",
                               "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load(path: str):
    """Load one build of k3_oracle.c and declare its C signatures."""
    L = ctypes.CDLL(path)
    L.orc_bf16_to_f64.argtypes = [_u16p, _i64, _f64p]
    L.orc_linear.argtypes = [_f64p, _i64, _int, _int, _u16p, _int, _f64p, _i64]
    L.orc_router_logits.argtypes = [_f64p, _i64, _int, _int, _u16p, ctypes.c_void_p, _int,
                                    _f32p]
    L.orc_topk_softmax.argtypes = [_f32p, _int, _int, _int, _i32p, _f64p]
    L.orc_shared_expert.argtypes = [_f64p, _i64, _int, _int, _u16p, _u16p, _int, _int, _f64p]
    L.orc_moe_experts.argtypes = [_f64p, _i64, _int, _int, _i32p, _f64p, _int,
                                  ctypes.c_void_p, ctypes.c_void_p, _int, _int, _int,
                                  ctypes.c_void_p, _f64p]
    L.orc_moe_experts.restype = _int
    L.orc_oproj_residual_rmsnorm.argtypes = [_f64p, _i64, _int, _int, _u16p, _int, _f64p,
                                             _f64p, ctypes.c_double, _f64p, _f64p]
    L.orc_max_threads.restype = _int
    L.orc_set_threads.argtypes = [_int]
    return L


def lib():
    """The loaded oracle library (built first if it is missing or stale)."""
    global _lib
    if _lib is None:
        build(force=False)
        _lib = _load(_LIB)
    return _lib


@contextlib.contextmanager
def use_library(path: str):
    """Route every oracle call through another build of k3_oracle.c for the
    duration of the block (the pin tests use it to show that a planted
    mistake in the oracle's source makes some pin fail)."""
    global _lib
    saved = lib()
    _lib = _load(path)
    try:
        yield
    finally:
        _lib = saved


def threads() -> int:
    """Threads the oracle's parallel loops use on this thread (OMP_NUM_THREADS
    or all cores, unless set_threads changed it)."""
    return lib().orc_max_threads()


def set_threads(n: int) -> None:
    """Threads this calling thread's oracle calls use from now on (timing
    only; every result is the same for any thread count)."""
    lib().orc_set_threads(int(n))


# ---------------------------------------------------------------- marshalling
def bf16_bits(t) -> np.ndarray:
    """uint16 bit patterns of a bf16 torch tensor (or a uint16 array), C order."""
    if isinstance(t, np.ndarray):
        assert t.dtype == np.uint16
        return np.ascontiguousarray(t)
    import torch
    assert t.dtype == torch.bfloat16, t.dtype
    return np.ascontiguousarray(t.detach().cpu().contiguous().view(torch.int16).numpy()
                                .view(np.uint16))


def widen(t) -> np.ndarray:
    """Exact fp64 values of a bf16 tensor (torch bf16 or uint16 bits)."""
    bits = bf16_bits(t)
    out = np.empty(bits.shape, dtype=np.float64)
    lib().orc_bf16_to_f64(bits.reshape(-1), bits.size, out.reshape(-1))
    return out


def _f64(a) -> np.ndarray:
    if not isinstance(a, np.ndarray):
        import torch
        if a.dtype == torch.bfloat16:
            return widen(a)
        a = a.detach().cpu().double().numpy()
    return np.ascontiguousarray(a, dtype=np.float64)


# ---------------------------------------------------------------- the steps
def linear(x, W) -> np.ndarray:
    """y = x . W^T for W [N x K] bf16; x [b x K] (fp64 or bf16)."""
    x = _f64(x)
    Wb = bf16_bits(W)
    b, K = x.shape
    N = Wb.shape[0]
    assert Wb.shape == (N, K)
    y = np.empty((b, N), dtype=np.float64)
    lib().orc_linear(x, K, b, K, Wb, N, y, N)
    return y


def router_logits(x, Wr, bias=None) -> np.ndarray:
    """fp32 logits [b x E] = fp32(x . Wr^T) (+ fp32 bias)."""
    x = _f64(x)
    Wb = bf16_bits(Wr)
    b, d = x.shape
    E = Wb.shape[0]
    out = np.empty((b, E), dtype=np.float32)
    bias_arr = None
    if bias is not None:
        bias_arr = np.ascontiguousarray(np.asarray(
            bias.detach().cpu().numpy() if hasattr(bias, "detach") else bias, dtype=np.float32))
        assert bias_arr.shape == (E,)
    lib().orc_router_logits(x, d, b, d, Wb,
                            bias_arr.ctypes.data if bias_arr is not None else None, E, out)
    return out


def topk_softmax(logits, k):
    """(ids [b x k] int32, w [b x k] fp64): top-k by (logit desc, index asc),
    softmax over all experts renormalised over the selected k."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    b, E = logits.shape
    assert 1 <= k <= E
    ids = np.empty((b, k), dtype=np.int32)
    w = np.empty((b, k), dtype=np.float64)
    lib().orc_topk_softmax(logits, b, E, k, ids, w)
    return ids, w


def shared_expert(x, w13_s, w2_s) -> np.ndarray:
    """y_s [b x d_out] = SwiGLU(x) with the shared expert's weights."""
    x = _f64(x)
    W13 = bf16_bits(w13_s)
    W2 = bf16_bits(w2_s)
    b, din = x.shape
    I = W13.shape[0] // 2
    dout = W2.shape[0]
    assert W13.shape == (2 * I, din) and W2.shape == (dout, I)
    y = np.empty((b, dout), dtype=np.float64)
    lib().orc_shared_expert(x, din, b, din, W13, W2, I, dout, y)
    return y


def _expert_tables(ids, expert_weights, E):
    """Pointer tables for the experts that ids name. expert_weights(e) returns
    expert e's (w13 [2I x din], w2 [dout x I]) bf16 tensors."""
    keep = {}
    for e in sorted(set(int(v) for v in np.asarray(ids).reshape(-1))):
        if not 0 <= e < E:
            raise ValueError(f"expert id {e} out of range [0, {E})")
        w13, w2 = expert_weights(e)
        keep[e] = (bf16_bits(w13), bf16_bits(w2))
    t13 = (ctypes.c_void_p * E)()
    t2 = (ctypes.c_void_p * E)()
    for e, (a, c) in keep.items():
        t13[e] = a.ctypes.data
        t2[e] = c.ctypes.data
    return keep, t13, t2


def moe_experts(z, ids, w, expert_weights, E, y_add=None) -> np.ndarray:
    """y[t] = y_add[t] + sum_j w[t][j] * Expert_{ids[t][j]}(z_t)."""
    z = _f64(z)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float64)
    b, din = z.shape
    k = ids.shape[1]
    keep, t13, t2 = _expert_tables(ids, expert_weights, E)
    a13, a2 = next(iter(keep.values()))
    I = a13.shape[0] // 2
    dout = a2.shape[0]
    for a, c in keep.values():
        assert a.shape == (2 * I, din) and c.shape == (dout, I)
    y = np.empty((b, dout), dtype=np.float64)
    ya = None if y_add is None else _f64(y_add)
    rc = lib().orc_moe_experts(z, din, b, din, ids, w, k, t13, t2, E, I, dout,
                               ya.ctypes.data if ya is not None else None, y)
    if rc != 0:
        raise ValueError("orc_moe_experts: bad expert id or missing weights")
    return y


def moe_block(x, weights: dict, k: int, expert_weights=None) -> dict:
    """The whole MoE block on input x [b x d].

    weights: w_router [E x d], bias (fp32 [E] or None), w_lat [d_lat x d],
    w13 [E x 2I x d_lat], w2 [E x d x I], w13_s [2I_s x d], w2_s [d x I_s].
    expert_weights(e) may replace w13/w2 lookup (for weights held elsewhere).
    Returns logits, ids, w, z, y_s, y_r and y = y_s + y_r, all fp64 except
    logits (fp32) and ids (int32).
    """
    E = weights["w_router"].shape[0]
    if expert_weights is None:
        def expert_weights(e):
            return weights["w13"][e], weights["w2"][e]
    xf = _f64(x)
    logits = router_logits(xf, weights["w_router"], weights.get("bias"))
    ids, w = topk_softmax(logits, k)
    z = linear(xf, weights["w_lat"])
    y_s = shared_expert(xf, weights["w13_s"], weights["w2_s"])
    y_r = moe_experts(z, ids, w, expert_weights, E)
    return {"logits": logits, "ids": ids, "w": w, "z": z, "y_s": y_s, "y_r": y_r,
            "y": y_s + y_r}


def oproj_residual_rmsnorm(a, Wo, r, gamma, eps):
    """(h, y): h = r + a . Wo^T; y = h / sqrt(mean(h^2) + eps) * gamma."""
    a = _f64(a)
    Wb = bf16_bits(Wo)
    b, K = a.shape
    d = Wb.shape[0]
    rf = _f64(r)
    gf = _f64(gamma).reshape(-1)
    assert rf.shape == (b, d) and gf.shape == (d,)
    h = np.empty((b, d), dtype=np.float64)
    y = np.empty((b, d), dtype=np.float64)
    lib().orc_oproj_residual_rmsnorm(a, K, b, K, Wb, d, rf, gf, float(eps), h, y)
    return h, y


def chain(x, r, w_in, w_o, gamma, eps) -> dict:
    """Input projection q = x . W_in^T, a = q[:, :K_o], then h and y as in
    oproj_residual_rmsnorm (K_o = W_o's input width)."""
    q = linear(x, w_in)
    k_o = bf16_bits(w_o).shape[1]
    a = np.ascontiguousarray(q[:, :k_o])
    h, y = oproj_residual_rmsnorm(a, w_o, r, gamma, eps)
    return {"q": q, "a": a, "h": h, "y": y}
