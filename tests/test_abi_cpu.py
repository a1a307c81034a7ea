"""C-ABI checks that need no GPU: the library loads, exports every declared entry point, sizes
workspaces, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def m():
    import sparse_moe_layer_softmax_amd as m
    if not os.path.exists(m.LIB_PATH):
        from sparse_moe_layer_softmax_amd import build
        build.build()
    return m


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for need in ("moe_route", "moe_permute", "moe_expert_ffn", "moe_combine", "moe_layer_forward"):
        assert need in names


def test_library_exports_every_declared_symbol(m):
    lib = m.library()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", m.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (moe_[a-z0-9_]+)\b", out))
    assert set(_declared_functions()) <= exported
    assert set(m.EXPORTED) == set(_declared_functions())


def test_header_compiles_as_plain_c(tmp_path):
    src = tmp_path / "use.c"
    src.write_text('#include "moe.h"\nint main(void){ moe_shape s = {0}; return (int)moe_layer_workspace_size(&s); }\n')
    subprocess.run(["gcc", "-std=c99", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", "/opt/rocm/include", "-c", str(src), "-o", str(tmp_path / "use.o")],
                   check=True)


HY4 = dict(T=64, H=6144, E=256, K=8, I=2048, routed_scaling=2.827)


def test_workspace_sizes(m):
    s = m.Shape(**HY4)
    assert m.moe_route_workspace_size(s) > 0
    assert m.moe_permute_workspace_size(s) > 0
    assert m.moe_expert_ffn_workspace_size(s, 256, 512) >= 512 * 2048 * 2
    lay = m.moe_layer_workspace_layout(s)
    assert lay["total"] == m.moe_layer_workspace_size(s)
    offs = [lay[k] for k in ("logits", "topk_w", "topk_idx", "counts", "offsets", "row_to_slot",
                             "slot_to_row", "h", "y")]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert lay["y"] - lay["h"] >= (64 + 512) * 2048 * 2
    assert lay["total"] - lay["y"] >= (64 + 512) * 6144 * 2
    # invalid shapes size to zero
    assert m.moe_layer_workspace_size(m.Shape(**dict(HY4, K=300))) == 0


def _call_route(m, shape, ws=1, ws_bytes=1 << 30, x=16, wr=16):
    lib = m.library()
    s = ctypes.byref(shape.c()) if shape is not None else None
    return lib.moe_route(s, x, wr, None, None, 4096, 4096, ws if ws is None else 256 * ws,
                         ws_bytes, None)


@pytest.mark.parametrize("bad, code", [
    (dict(T=0), -1), (dict(H=0), -1), (dict(E=0), -1), (dict(K=0), -1), (dict(K=9, E=8), -1),
    (dict(n_shared=2), -1), (dict(routed_scaling=float("inf")), -1),
    (dict(K=17, E=64), -2), (dict(E=257), -2), (dict(H=6100), -2), (dict(I=2000), -2),
    (dict(T=1 << 28), -2),
])
def test_shape_errors_are_caught_on_the_host(m, bad, code):
    # the pointers below are never dereferenced: rejection happens before any launch
    assert _call_route(m, m.Shape(**dict(HY4, **bad))) == code


def test_null_and_workspace_errors(m):
    lib = m.library()
    s = m.Shape(**HY4)
    assert _call_route(m, None) == m.MOE_ERR_INVALID_ARG
    assert _call_route(m, s, x=None) == m.MOE_ERR_INVALID_ARG
    assert _call_route(m, s, ws=None) == m.MOE_ERR_INVALID_ARG
    assert _call_route(m, s, ws_bytes=16) == m.MOE_ERR_WORKSPACE
    # misaligned workspace
    assert lib.moe_route(ctypes.byref(s.c()), 16, 16, None, None, 16, 16, 256 + 8, 1 << 30, None) == m.MOE_ERR_WORKSPACE
    sc = ctypes.byref(s.c())
    assert lib.moe_permute(sc, 16, None, 16, 16, 16, 256, 1 << 30, None) == m.MOE_ERR_INVALID_ARG
    assert lib.moe_permute(sc, 16, 16, 16, 16, 16, 256, 8, None) == m.MOE_ERR_WORKSPACE
    # expert FFN: identity rows beyond T, several groups without offsets, group count bounds
    assert lib.moe_expert_ffn(sc, 1, 65, 16, None, None, 16, 16, 16, None, 16, 256, 1 << 30, None) == m.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_ffn(sc, 4, 64, 16, None, None, 16, 16, 16, None, 16, 256, 1 << 30, None) == m.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_ffn(sc, 0, 64, 16, None, 16, 16, 16, 16, None, 16, 256, 1 << 30, None) == m.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_ffn(sc, 1, 64, 16, None, None, 16, 16, 16, None, 16, 256, 64, None) == m.MOE_ERR_WORKSPACE
    # combine: unaligned rows
    assert lib.moe_combine(sc, 18, 16, 16, None, 16, None) == m.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(sc, None, 16, 16, None, 16, None) == m.MOE_ERR_INVALID_ARG
    # layer: shared expert pointers must match n_shared
    lf = lib.moe_layer_forward
    assert lf(sc, 16, 16, None, 16, 16, 16, None, None, None, 16, 256, 1 << 40, None) == m.MOE_ERR_INVALID_ARG
    s0 = ctypes.byref(m.Shape(**dict(HY4, n_shared=0)).c())
    assert lf(s0, 16, 16, None, 16, 16, 16, 16, 16, 16, 16, 256, 1 << 40, None) == m.MOE_ERR_INVALID_ARG
    assert lf(sc, 16, 16, None, 16, 16, 16, 16, 16, 16, 16, 256, 1024, None) == m.MOE_ERR_WORKSPACE
    assert m.strerror(m.MOE_ERR_WORKSPACE).startswith("workspace")
    assert m.strerror(12345) == "unknown error"


def test_binding_raises_on_errors(m):
    s = m.Shape(**dict(HY4, K=0))
    with pytest.raises(m.MoeError) as ei:
        m.moe_combine(s, 16, 16, 16, None, 16, stream=0)
    assert ei.value.code == m.MOE_ERR_INVALID_ARG


def test_fp8_entry_point_errors(m):
    lib = m.library()
    sc = ctypes.byref(m.Shape(**HY4).c())
    ffn8 = lib.moe_expert_ffn_fp8
    # codes without their scales, or scales without codes
    assert ffn8(sc, 1, 64, 16, None, None, 16, None, 16, 16, 16, 16, 16, 16, 256, 1 << 30, None) == m.MOE_ERR_INVALID_ARG
    assert ffn8(sc, 1, 64, 16, None, None, 16, 16, 16, 16, None, 16, 16, 16, 256, 1 << 30, None) == m.MOE_ERR_INVALID_ARG
    assert ffn8(sc, 1, 64, 16, None, None, 16, 16, 16, 16, 16, 16, 16, 16, 256, 64, None) == m.MOE_ERR_WORKSPACE
    lf8 = lib.moe_layer_forward_fp8
    w = [16] * 6
    # shared expert present (n_shared = 1) but one shared scale missing
    assert lf8(sc, 16, 16, None, *w, 16, 16, 16, None, 16, 16, 16, 256, 1 << 40, None, None) == m.MOE_ERR_INVALID_ARG
    # no shared expert, yet a shared pointer given
    s0 = ctypes.byref(m.Shape(**dict(HY4, n_shared=0)).c())
    assert lf8(s0, 16, 16, None, *w, None, None, None, None, None, 16, 16, 256, 1 << 40, None, None) == m.MOE_ERR_INVALID_ARG
    assert lf8(sc, 16, 16, None, *w, *w, 16, 256, 1024, None, None) == m.MOE_ERR_WORKSPACE
    assert lf8(sc, 16, 16, None, *w[:5], None, *w, 16, 256, 1 << 40, None, None) == m.MOE_ERR_INVALID_ARG


def test_route_train_errors(m):
    lib = m.library()
    s = m.Shape(**HY4)
    sc = ctypes.byref(s.c())
    assert m.moe_route_train_workspace_size(s) > m.moe_route_workspace_size(s)
    n = m.moe_route_train_workspace_size(s)
    rt = lib.moe_route_train
    ok = [16, 16, None, None, None, 16, 16, 16, 16, 16, None, None]
    assert rt(sc, *ok, 0.9, 256, n - 1, None) == m.MOE_ERR_WORKSPACE
    bad = list(ok)
    bad[9] = None  # aux_loss
    assert rt(sc, *bad, 0.9, 256, n, None) == m.MOE_ERR_INVALID_ARG
    assert rt(sc, *ok, 1.5, 256, n, None) == m.MOE_ERR_INVALID_ARG
    assert rt(sc, *ok, float("nan"), 256, n, None) == m.MOE_ERR_INVALID_ARG
    assert rt(sc, *ok, 0.9, 256 + 8, n, None) == m.MOE_ERR_WORKSPACE  # misaligned


def test_binding_argument_counts_match_the_header(m):
    """Each ctypes signature has as many parameters as the header's declaration."""
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    lib = m.library()
    for name in _declared_functions():
        decl = re.search(r"\b%s\s*\(([^)]*)\)" % name, src).group(1)
        n = 0 if decl.strip() in ("", "void") else decl.count(",") + 1
        fn = getattr(lib, name)
        assert fn.argtypes is not None and len(fn.argtypes) == n, (name, n, fn.argtypes)


# The LDS-tiled MFMA kernel reaches operand rows through 32-bit offsets in 16-byte units, so no
# operand it reads may pass 64 GiB; the host rejects larger shapes (MOE_ERR_UNSUPPORTED) before
# any launch. The thresholds below are the exact largest token counts at the Hy4 shape.
FWD_T_MAX = (1 << 36) // (2 * 9 * 2048)   # h [T*(K+1), I] bf16 at K = 8, I = 2048


def _bwd_t_max(H=6144, I=2048, E=256, K=8):
    def fits(T):
        rows = T * (K + 1)
        ld = ((rows + 63) // 64 + E + 1) * 64  # row-contiguous copies of the weight gradients
        lim = 1 << 36
        return rows * H * 2 <= lim and rows * 2 * I * 2 <= lim and H * ld * 2 <= lim and 2 * I * ld * 2 <= lim
    lo, hi = 1, 1 << 24
    while lo < hi:
        mid = (lo + hi + 1) // 2
        lo, hi = (mid, hi) if fits(mid) else (lo, mid - 1)
    return lo


def test_operand_size_limit_forward(m):
    assert FWD_T_MAX == 1864135  # the figure the header states
    ok = m.Shape(**dict(HY4, T=FWD_T_MAX))
    big = m.Shape(**dict(HY4, T=FWD_T_MAX + 1))
    assert m.moe_layer_workspace_size(ok) > 0
    assert m.moe_layer_workspace_size(big) == 0
    assert _call_route(m, big) == m.MOE_ERR_UNSUPPORTED
    assert _call_route(m, ok) != m.MOE_ERR_UNSUPPORTED
    # moe_expert_ffn checks its own row bound: rows_max * I * 2 bytes <= 64 GiB
    s = m.Shape(**dict(HY4, T=1 << 20, K=1))
    rmax = (1 << 36) // (2 * 2048)
    assert m.moe_expert_ffn_workspace_size(s, 1, rmax) > 0
    lib = m.library()
    sc = ctypes.byref(s.c())
    args = (16, 16, 16, 16, 16, 16, None, 16, 256, 1 << 60, None)
    assert lib.moe_expert_ffn(sc, 1, rmax + 1, *args) == m.MOE_ERR_UNSUPPORTED
    # x [T, H] alone past 64 GiB
    wide = m.Shape(**dict(HY4, T=(1 << 36) // (2 * 6144) + 1, K=1, E=1, n_shared=0))
    assert m.moe_layer_workspace_size(wide) == 0


def test_operand_size_limit_backward(m):
    tb = _bwd_t_max()
    assert tb == 619548  # the figure the header states
    assert m.moe_layer_backward_workspace_size(m.Shape(**dict(HY4, T=tb))) > 0
    assert m.moe_layer_backward_workspace_size(m.Shape(**dict(HY4, T=tb + 1))) == 0
    # the forward alone still accepts that size
    assert m.moe_layer_workspace_size(m.Shape(**dict(HY4, T=tb + 1))) > 0
    lib = m.library()
    sc = ctypes.byref(m.Shape(**dict(HY4, T=tb + 1)).c())
    rc = lib.moe_layer_backward(sc, 16, 16, 16, 16, 16, 16, 16, 16, 256, 1 << 60, None, 16, 0.0,
                                16, 16, 16, 16, 16, 16, 16, 16, None, None, 256, 1 << 60, None)
    assert rc == m.MOE_ERR_UNSUPPORTED
