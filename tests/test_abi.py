"""Host-side checks of the C ABI (no GPU needed): libk3dec loads, exports
every function include/k3dec.h declares, and each entry point rejects bad
arguments with the documented status before launching anything."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "k3dec.h")

K3_OK, INVALID, UNSUP, WORKSPACE = 0, -1, -2, -3
P = 1 << 20           # a fake, 16-byte aligned address (never dereferenced)
MIS = (1 << 20) + 8   # a fake misaligned address


@pytest.fixture(scope="module")
def L():
    import moe_router_topk_amd as k3
    return k3.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(k3_\w+)\s*\(", text)))


def test_header_compiles_as_c():
    src = f'#include "{HEADER}"\nint main(void) {{ return K3_OK; }}\n'
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-x", "c", "-fsyntax-only", "-"],
                   input=src, text=True, check=True)


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 15
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing
    import moe_router_topk_amd as k3
    assert set(k3.EXPORTED_SYMBOLS) == set(names)


def test_exports_no_cxx_or_torch_types():
    """nm: the dynamic symbols named k3_* are plain C names."""
    import moe_router_topk_amd as k3
    out = subprocess.run(["nm", "-D", "--defined-only", k3.library_path()],
                         capture_output=True, text=True, check=True).stdout
    k3_syms = [ln.split()[-1] for ln in out.splitlines() if " k3_" in ln]
    assert k3_syms and all(re.fullmatch(r"k3_\w+", s) for s in k3_syms)


def test_status_strings(L):
    L.k3_status_string.restype = ctypes.c_char_p
    for code in (0, -1, -2, -3, -4, -5):
        s = L.k3_status_string(code).decode()
        assert s.startswith("K3_"), s
    assert L.k3_status_string(-99).decode() == "unknown k3 status"
    assert L.k3_version() == 10000


def test_force_variant_validation(L):
    assert L.k3_force_variant(1, 2) == K3_OK
    assert L.k3_force_variant(1, 0) == K3_OK
    assert L.k3_force_variant(7, 2) == K3_OK
    assert L.k3_force_variant(7, 0) == K3_OK
    assert L.k3_force_variant(6, 1) == K3_OK
    assert L.k3_force_variant(6, 0) == K3_OK
    assert L.k3_force_variant(8, 2) == K3_OK  # the expert engine
    assert L.k3_force_variant(8, 0) == K3_OK
    assert L.k3_force_variant(9, 0) == INVALID  # the dense pass record cannot be forced
    assert L.k3_force_variant(10, 0) == INVALID
    assert L.k3_force_variant(1, 17) == INVALID
    assert L.k3_force_variant(1, 6) == INVALID  # record-only variants
    assert L.k3_force_variant(0, 6) == INVALID


def test_router_last_workgroup_variant_is_batch_one_only(L):
    """The forced last-workgroup router runs one token only; other batches
    and other ops refuse it before launching anything."""
    assert L.k3_force_variant(0, 5) == K3_OK
    try:
        assert _router(L, b=2) == UNSUP
    finally:
        assert L.k3_force_variant(0, 0) == K3_OK
    assert L.k3_force_variant(1, 5) == K3_OK
    try:
        assert L.k3_proj_skinny(P, 256, 1, 256, P, 256, P, 256, P, 1 << 20, None) == UNSUP
    finally:
        assert L.k3_force_variant(1, 0) == K3_OK


def test_op_and_variant_codes_match_header():
    """The binding's op and variant tables carry the header's values."""
    import moe_router_topk_amd as k3
    text = open(HEADER).read()
    ops = {m.group(1).lower(): int(m.group(2))
           for m in re.finditer(r"#define K3_OP_(\w+) (\d+)", text)}
    variants = {m.group(1).lower(): int(m.group(2))
                for m in re.finditer(r"#define K3_VARIANT_(\w+) (\d+)", text)}
    assert ops == k3.OP
    assert variants == k3.VARIANT


def test_workspace_sizes(L):
    import moe_router_topk_amd as k3
    assert k3.workspace_size("router_topk", b=64, E=384) >= 64 * 384 * 4
    assert k3.workspace_size("proj_skinny", b=64, K=7168, N=12288) >= 4 * 64 * 12288 * 4
    assert k3.workspace_size("router_topk_latent", b=64, E=384, d_lat=7168) >= \
        k3.workspace_size("router_topk", b=64, E=384) + 4 * 64 * 7168 * 4
    assert k3.workspace_size("moe_block", b=64, d=7168, E=384, k=8, d_lat=7168, I=2048,
                             I_s=2048) >= 4 * 64 * (384 + 7168 + 4096) * 4
    assert k3.workspace_size("moe_experts", b=64, d_in=7168, E=384, k=8, I=2048,
                             d_out=7168) >= 512 * 2048 * 2 + 512 * 7168 * 4
    assert k3.workspace_size("shared_expert", b=64, d=7168, I=2048) >= 64 * 2048 * 2
    assert k3.workspace_size("oproj_residual", b=64, K=8192, d=7168) >= 64 * 7168 * 4
    assert k3.workspace_size("router_topk", b=0, E=384) == 0


def _router(L, **kw):
    a = dict(x=P, ldx=256, b=1, d=256, w=P, bias=None, E=8, k=2, ids=P, wts=P, ws=P,
             wsb=1 << 20, stream=None)
    a.update(kw)
    return L.k3_router_topk(a["x"], a["ldx"], a["b"], a["d"], a["w"], a["bias"], a["E"], a["k"],
                            a["ids"], a["wts"], a["ws"], a["wsb"], a["stream"])


def test_router_topk_validation(L):
    assert _router(L, x=None) == INVALID
    assert _router(L, b=0) == INVALID
    assert _router(L, ldx=128) == INVALID
    assert _router(L, b=65) == UNSUP
    assert _router(L, k=9) == UNSUP
    assert _router(L, E=1025, k=2) == UNSUP
    assert _router(L, k=33, E=64) == UNSUP
    assert _router(L, d=250, ldx=256) == UNSUP
    assert _router(L, x=MIS) == UNSUP
    assert _router(L, ws=None) == WORKSPACE
    assert _router(L, wsb=16) == WORKSPACE


def _router_latent(L, **kw):
    a = dict(x=P, ldx=256, b=1, d=256, w=P, bias=None, E=8, k=2, wl=P, dl=256, ids=P, wts=P,
             z=P, ldz=256, ws=P, wsb=1 << 20)
    a.update(kw)
    return L.k3_router_topk_latent(a["x"], a["ldx"], a["b"], a["d"], a["w"], a["bias"], a["E"],
                                   a["k"], a["wl"], a["dl"], a["ids"], a["wts"], a["z"], a["ldz"],
                                   a["ws"], a["wsb"], None)


def test_router_topk_latent_validation(L):
    assert _router_latent(L, wl=None) == INVALID
    assert _router_latent(L, z=None) == INVALID
    assert _router_latent(L, ldz=128) == INVALID
    assert _router_latent(L, dl=0) == INVALID
    assert _router_latent(L, x=None) == INVALID
    assert _router_latent(L, b=65) == UNSUP
    assert _router_latent(L, wl=MIS) == UNSUP
    assert _router_latent(L, k=9) == UNSUP
    assert _router_latent(L, ws=None) == WORKSPACE
    # the router-only workspace is too small once the latent rows join the pass
    small = L.k3_router_topk_workspace_size(64, 8)
    assert _router_latent(L, b=64, wsb=small) == WORKSPACE


def _block(L, **kw):
    a = dict(x=P, ldx=256, b=1, d=256, wr=P, bias=None, E=8, k=2, wl=P, dl=256, w13=P, w2=P,
             I=128, w13s=P, w2s=P, Is=128, ids=P, wts=P, z=P, ldz=256, ys=P, y=P, ws=P,
             wsb=1 << 24)
    a.update(kw)
    return L.k3_moe_block(a["x"], a["ldx"], a["b"], a["d"], a["wr"], a["bias"], a["E"], a["k"],
                          a["wl"], a["dl"], a["w13"], a["w2"], a["I"], a["w13s"], a["w2s"],
                          a["Is"], a["ids"], a["wts"], a["z"], a["ldz"], a["ys"], a["y"],
                          a["ws"], a["wsb"], None)


def test_moe_block_validation(L):
    assert _block(L, y=None) == INVALID
    assert _block(L, ys=None) == INVALID
    assert _block(L, Is=0) == INVALID
    assert _block(L, ldz=128) == INVALID
    assert _block(L, b=65) == UNSUP
    assert _block(L, I=100) == UNSUP
    assert _block(L, Is=200) == UNSUP
    assert _block(L, d=200, ldx=256) == UNSUP
    assert _block(L, w2s=MIS) == UNSUP
    assert _block(L, k=9) == UNSUP
    assert _block(L, ws=None) == WORKSPACE
    assert _block(L, wsb=4096) == WORKSPACE


def _proj(L, **kw):
    a = dict(x=P, ldx=256, b=1, K=256, w=P, N=64, y=P, ldy=64)
    a.update(kw)
    return L.k3_proj_skinny(a["x"], a["ldx"], a["b"], a["K"], a["w"], a["N"], a["y"], a["ldy"],
                            None, 0, None)


def test_proj_skinny_validation(L):
    assert _proj(L, w=None) == INVALID
    assert _proj(L, N=0) == INVALID
    assert _proj(L, ldy=32) == INVALID
    assert _proj(L, b=65) == UNSUP
    assert _proj(L, K=252, ldx=256) == UNSUP
    assert _proj(L, w=MIS) == UNSUP
    # above 4 tokens the split-K MFMA variant keeps its partial sums in the workspace
    assert _proj(L, b=16, K=264, ldx=264) == WORKSPACE
    assert L.k3_force_variant(1, 1) == K3_OK
    try:
        assert _proj(L, b=9) == UNSUP
    finally:
        L.k3_force_variant(1, 0)


def _moe(L, **kw):
    a = dict(z=P, ldz=256, b=1, d_in=256, ids=P, w=P, k=2, w13=P, w2=P, E=8, I=128, d_out=256,
             y_add=None, ev=None, y=P, cu=0, ws=P, wsb=1 << 24)
    a.update(kw)
    return L.k3_moe_experts(a["z"], a["ldz"], a["b"], a["d_in"], a["ids"], a["w"], a["k"],
                            a["w13"], a["w2"], a["E"], a["I"], a["d_out"], a["y_add"], a["ev"],
                            a["y"], a["cu"], a["ws"], a["wsb"], None)


def test_moe_experts_validation(L):
    assert _moe(L, y=None) == INVALID
    assert _moe(L, cu=-1) == INVALID
    assert _moe(L, ldz=8) == INVALID
    assert _moe(L, b=65) == UNSUP
    assert _moe(L, k=33) == UNSUP
    assert _moe(L, I=96) == UNSUP
    assert _moe(L, d_in=200, ldz=256) == UNSUP
    assert _moe(L, d_out=250) == UNSUP
    assert _moe(L, w2=MIS) == UNSUP
    assert _moe(L, ws=None) == WORKSPACE
    assert _moe(L, wsb=1024) == WORKSPACE


def _shared(L, **kw):
    a = dict(x=P, ldx=256, b=1, d=256, w13=P, w2=P, I=128, y=P, cu=0, ws=P, wsb=1 << 20)
    a.update(kw)
    return L.k3_shared_expert(a["x"], a["ldx"], a["b"], a["d"], a["w13"], a["w2"], a["I"],
                              a["y"], a["cu"], a["ws"], a["wsb"], None)


def test_shared_expert_validation(L):
    assert _shared(L, w13=None) == INVALID
    assert _shared(L, I=0) == INVALID
    assert _shared(L, b=65) == UNSUP
    assert _shared(L, d=192, ldx=256) == UNSUP
    assert _shared(L, x=MIS) == UNSUP
    assert _shared(L, wsb=8) == WORKSPACE


def _oproj(L, **kw):
    a = dict(a=P, lda=512, b=1, K=256, w=P, d=256, r=P, g=P, eps=1e-6, y=P, ws=P, wsb=1 << 20)
    a.update(kw)
    L.k3_oproj_residual.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    return L.k3_oproj_residual(a["a"], a["lda"], a["b"], a["K"], a["w"], a["d"], a["r"], a["g"],
                               a["eps"], a["y"], a["ws"], a["wsb"], None)


def test_oproj_residual_validation(L):
    assert _oproj(L, g=None) == INVALID
    assert _oproj(L, eps=-1.0) == INVALID
    assert _oproj(L, eps=float("nan")) == INVALID
    assert _oproj(L, lda=128) == INVALID
    assert _oproj(L, b=65) == UNSUP
    assert _oproj(L, d=250) == UNSUP
    assert _oproj(L, a=MIS) == UNSUP
    assert _oproj(L, ws=None) == WORKSPACE


def test_prefetch_validation(L):
    assert L.k3_prefetch(P, 0, 0, None) == K3_OK  # nothing to read: no launch
    assert L.k3_prefetch(None, 16, 0, None) == INVALID
    assert L.k3_prefetch(P, 16, -1, None) == INVALID
    assert L.k3_prefetch(MIS, 16, 0, None) == UNSUP
    assert L.k3_prefetch(P, 24, 0, None) == UNSUP


def test_stream_read_validation(L):
    assert L.k3_stream_read(P, 0, None) == K3_OK  # nothing to read: no launch
    assert L.k3_stream_read(None, 16, None) == INVALID
    assert L.k3_stream_read(MIS, 16, None) == UNSUP
    assert L.k3_stream_read(P, 24, None) == UNSUP


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    import moe_router_topk_amd as k3
    monkeypatch.setattr(k3, "_lib", None)
    monkeypatch.setattr(k3, "_LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        k3.lib()


def test_noalloc_argument_checks(L):
    """k3_moe_block_noalloc rejects a NULL input and shapes beyond its static
    scratch before it touches the device (fake pointers are never used)."""
    f = L.k3_moe_block_noalloc
    f.restype = ctypes.c_int
    v, i64 = ctypes.c_void_p, ctypes.c_int64
    f.argtypes = [v, i64, ctypes.c_int, ctypes.c_int, v, v, ctypes.c_int, ctypes.c_int, v,
                  ctypes.c_int, v, v, ctypes.c_int, v, v, ctypes.c_int, v, v, v, i64, v, v, v]

    def call(x, b, d, E, k, d_lat, I, I_s):
        return f(x, d, b, d, P, None, E, k, P, d_lat, P, P, I, P, P, I_s, P, P, P, d_lat, P, P,
                 None)

    assert call(None, 1, 7168, 384, 8, 7168, 2048, 2048) == INVALID
    assert call(P, 0, 7168, 384, 8, 7168, 2048, 2048) == INVALID
    # 64 tokens at E = 1024, top-32, d = I = 8192 need about 122 MiB of scratch
    assert call(P, 64, 8192, 1024, 32, 8192, 8192, 8192) == -5
    L.k3_status_string.restype = ctypes.c_char_p
    assert b"K3_NOALLOC_SCRATCH_BYTES" in L.k3_status_string(-5)
