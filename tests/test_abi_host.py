"""C ABI checks that need no GPU: the library loads, exports exactly what include/wbmm.h declares,
the Python binding's signatures match the header, and invalid arguments are rejected on the host
(every call here returns before anything is enqueued)."""
import ctypes
import os
import re
import subprocess

import pytest

import receptive_field_spatial_amd as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wbmm.h")

FAKE = 0x100000          # an aligned non-NULL address; never dereferenced by these calls
FAKE2 = 0x200000


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(R.lib_path()):
        from receptive_field_spatial_amd.build import build
        build(verbose=False)
    return R.load_library()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    decls = re.findall(r"^\s*(?:wbmm_status|int|size_t|double|const char\*)\s+(wbmm_\w+)\s*\(([^;]*?)\)\s*;",
                       text, flags=re.M | re.S)
    out = {}
    for name, params in decls:
        params = params.strip()
        out[name] = 0 if params in ("", "void") else len([p for p in params.split(",") if p.strip()])
    return out


def test_header_declares_the_entry_points():
    fns = header_functions()
    for name in ["wbmm_build_index", "wbmm_build_matrix", "wbmm_fold_hier", "wbmm_forward",
                 "wbmm_backward", "wbmm_forward_workspace_bytes", "wbmm_backward_workspace_bytes",
                 "wbmm_last_error", "wbmm_abi_version", "wbmm_forward_hier", "wbmm_backward_hier",
                 "wbmm_dwconv_forward", "wbmm_forward_shifted", "wbmm_backward_shifted",
                 "wbmm_backward_bf16", "wbmm_probe_mfma"]:
        assert name in fns, name


def test_library_exports_exactly_the_header(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", R.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l and l.split()[-1].startswith("wbmm_")}
    assert exported == set(header_functions())
    for name in exported:
        assert hasattr(lib, name)


def test_binding_signatures_match_header(lib):
    for name, nparams in header_functions().items():
        assert len(getattr(lib, name).argtypes) == nparams, name


def test_abi_version(lib):
    assert lib.wbmm_abi_version() == 1


def err(lib):
    return lib.wbmm_last_error().decode()


def test_build_index_validation(lib):
    assert lib.wbmm_build_index(0, FAKE, None) == R.WBMM_E_INVALID
    assert "w=0" in err(lib)
    assert lib.wbmm_build_index(33, FAKE, None) == R.WBMM_E_INVALID
    assert lib.wbmm_build_index(7, None, None) == R.WBMM_E_INVALID
    assert lib.wbmm_build_index(7, FAKE + 2, None) == R.WBMM_E_UNSUPPORTED


def test_build_matrix_validation(lib):
    assert lib.wbmm_build_matrix(FAKE, 0, 7, 0, FAKE2, None) == R.WBMM_E_INVALID
    assert lib.wbmm_build_matrix(FAKE, 4, 7, 5, FAKE2, None) == R.WBMM_E_INVALID
    assert lib.wbmm_build_matrix(None, 4, 7, 0, FAKE2, None) == R.WBMM_E_INVALID
    assert lib.wbmm_build_matrix(FAKE, 4, 7, 0, FAKE + 4, None) == R.WBMM_E_INVALID  # overlap
    assert "overlaps" in err(lib)


def test_fold_validation(lib):
    for w, s in [(14, 5), (14, 14), (14, 0), (7, 7)]:
        assert lib.wbmm_fold_hier(FAKE, FAKE2, 2, w, s, 0, FAKE, None) == R.WBMM_E_INVALID, (w, s)
    assert lib.wbmm_fold_hier(FAKE, FAKE2, 2, 14, 7, 0, FAKE + 8, None) == R.WBMM_E_INVALID


def fwd(lib, **kw):
    a = dict(B=1, C=2, H=8, W=8, w=4, layout=0, ind=0, outd=0, x=FAKE, T=FAKE2, M=None, mix=None,
             z=None, y=0x400000, ws=None, wsb=0)
    a.update(kw)
    return lib.wbmm_forward(a["B"], a["C"], a["H"], a["W"], a["w"], a["layout"], a["ind"],
                            a["outd"], a["x"], a["T"], a["M"], a["mix"], a["z"], a["y"], a["ws"],
                            a["wsb"], None)


def test_forward_validation(lib):
    assert fwd(lib, w=0) == R.WBMM_E_INVALID
    assert fwd(lib, w=33) == R.WBMM_E_INVALID
    assert fwd(lib, B=0) == R.WBMM_E_INVALID
    assert fwd(lib, layout=3) == R.WBMM_E_INVALID
    assert fwd(lib, ind=7) == R.WBMM_E_INVALID
    assert fwd(lib, T=None) == R.WBMM_E_INVALID                 # neither T nor M
    assert fwd(lib, M=0x800000) == R.WBMM_E_INVALID             # both T and M
    assert "exactly one" in err(lib)
    assert fwd(lib, x=None) == R.WBMM_E_INVALID
    assert fwd(lib, y=FAKE) == R.WBMM_E_INVALID                 # y aliases x
    # bf16 output with the mix is supported (y and z_save rounded from the fp32 pre-mix map)
    assert lib.wbmm_forward_workspace_bytes(2, 3, 128, 128, 14, 0, 1, 1) > 0  # window mode, z_save
    assert fwd(lib, x=FAKE + 2) == R.WBMM_E_UNSUPPORTED         # misaligned fp32
    assert fwd(lib, C=70000) == R.WBMM_E_UNSUPPORTED


def test_forward_workspace_rules(lib):
    # a mix on images too large for one workgroup needs an fp32 z buffer unless z_save is given
    need = lib.wbmm_forward_workspace_bytes(1, 2, 128, 128, 14, 0, 1, 0)
    assert need == 1 * 2 * 128 * 128 * 4
    # with z_save the fp32 call writes z there, but a bf16 z_save takes the fp32 map through the
    # workspace: the query (which has no dtype argument) reports the larger need
    assert lib.wbmm_forward_workspace_bytes(1, 2, 128, 128, 14, 0, 1, 1) == need
    # with a table the mix is fused in-kernel here (64 windows per image; the fast fp32 and bf16
    # w = 14 kernels), but the query also covers a cached matrix, whose fast fp32 kernel writes
    # the pre-mix map to the workspace for a separate mix pass
    assert lib.wbmm_forward_workspace_bytes(1, 2, 100, 100, 14, 0, 1, 0) == 1 * 2 * 100 * 100 * 4
    assert lib.wbmm_forward_workspace_bytes(64, 192, 28, 28, 14, 0, 1, 0) == 64 * 192 * 28 * 28 * 4
    # the fast w = 7 shape (bf16 and fp32 kernels) keeps z in the workspace for its separate mix
    # pass: the fp32 map is the larger need
    assert lib.wbmm_forward_workspace_bytes(8, 4, 56, 56, 7, 0, 1, 0) == 8 * 4 * 56 * 56 * 4
    # with z_save the fp32 pre-mix map goes there
    assert lib.wbmm_forward_workspace_bytes(64, 192, 28, 28, 14, 0, 1, 1) == 0
    # the fast fp32 w = 28 kernel (56x56 maps) runs the mix as its own pass too
    assert lib.wbmm_forward_workspace_bytes(3, 2, 56, 56, 28, 0, 1, 0) == 3 * 2 * 56 * 56 * 4
    assert lib.wbmm_forward_workspace_bytes(3, 2, 56, 56, 28, 0, 0, 0) == 0
    assert lib.wbmm_forward_workspace_bytes(1, 2, 8, 8, 0, 0, 0, 0) == 0       # invalid -> 0
    st = fwd(lib, B=1, C=2, H=128, W=128, w=14, mix=0x900000, y=0x40000000, ws=None, wsb=0)
    assert st == R.WBMM_E_WORKSPACE
    st = fwd(lib, B=1, C=2, H=128, W=128, w=14, mix=0x900000, y=0x40000000, ws=0xA00000, wsb=need - 1)
    assert st == R.WBMM_E_WORKSPACE


def bwd(lib, **kw):
    a = dict(B=1, C=2, H=8, W=8, w=4, layout=0, x=FAKE, T=FAKE2, M=None, mix=None, z=None,
             dy=0x300000, dx=0x400000, dT=0x500000, dW=None, ws=None, wsb=0)
    a.update(kw)
    return lib.wbmm_backward(a["B"], a["C"], a["H"], a["W"], a["w"], a["layout"], a["x"], a["T"],
                             a["M"], a["mix"], a["z"], a["dy"], a["dx"], a["dT"], a["dW"], a["ws"],
                             a["wsb"], None)


def test_backward_validation(lib):
    assert bwd(lib, w=33) == R.WBMM_E_INVALID
    assert "w=33" in err(lib)
    # 16 < w <= 32: the wide-window backward, which needs a workspace
    assert bwd(lib, w=17) == R.WBMM_E_WORKSPACE
    assert bwd(lib, T=None) == R.WBMM_E_INVALID
    assert bwd(lib, mix=0x900000) == R.WBMM_E_INVALID           # mix without z_saved
    assert bwd(lib, z=0x900000) == R.WBMM_E_INVALID             # z_saved without mix
    assert bwd(lib, dx=FAKE) == R.WBMM_E_INVALID                # dx aliases x
    assert bwd(lib, dy=None) == R.WBMM_E_INVALID
    need = lib.wbmm_backward_workspace_bytes(1, 2, 8, 8, 4, 0, 0)
    assert need > 0
    assert bwd(lib) == R.WBMM_E_WORKSPACE
    assert bwd(lib, ws=0xA00000, wsb=need - 1) == R.WBMM_E_WORKSPACE
    assert bwd(lib, ws=0xA00010, wsb=need) == R.WBMM_E_UNSUPPORTED  # not 256-byte aligned
    assert lib.wbmm_backward_workspace_bytes(1, 2, 8, 8, 17, 0, 0) > 0
    assert lib.wbmm_backward_workspace_bytes(1, 2, 8, 8, 33, 0, 0) == 0


def hier_fwd(lib, **kw):
    a = dict(B=1, C=2, H=28, W=28, w=14, s=7, layout=0, x=FAKE, T=FAKE2, Ts=0x300000, mix=None,
             z=None, y=0x40000000, ws=None, wsb=0)
    a.update(kw)
    return lib.wbmm_forward_hier(a["B"], a["C"], a["H"], a["W"], a["w"], a["s"], a["layout"],
                                 a["x"], a["T"], a["Ts"], a["mix"], a["z"], a["y"], a["ws"],
                                 a["wsb"], None)


def hier_bwd(lib, **kw):
    a = dict(B=1, C=2, H=28, W=28, w=14, s=7, layout=0, x=FAKE, T=FAKE2, Ts=0x300000, mix=None,
             z=None, dy=0x380000, dx=0x400000, dT=0x500000, dTs=0x580000, dW=None, ws=None, wsb=0)
    a.update(kw)
    return lib.wbmm_backward_hier(a["B"], a["C"], a["H"], a["W"], a["w"], a["s"], a["layout"],
                                  a["x"], a["T"], a["Ts"], a["mix"], a["z"], a["dy"], a["dx"],
                                  a["dT"], a["dTs"], a["dW"], a["ws"], a["wsb"], None)


def test_hier_validation(lib):
    """The hierarchical entry points: s divides w and s < w, both tables required, fp32 maps
    checked like the plain calls, workspace sizes reported and enforced. Sub-windows other than
    the quadrants (and w = 2s above 16) need the folded matrix in the workspace: C w^4 floats
    at least."""
    for w, s in [(14, 14), (14, 0), (14, 5), (12, 13), (14, -7)]:
        assert hier_fwd(lib, w=w, s=s) == R.WBMM_E_INVALID, (w, s)
        assert hier_bwd(lib, w=w, s=s) == R.WBMM_E_INVALID, (w, s)
        assert lib.wbmm_forward_hier_workspace_bytes(1, 2, 28, 28, w, s, 0, 1, 0) == 0
        assert lib.wbmm_backward_hier_workspace_bytes(1, 2, 28, 28, w, s, 0, 0) == 0
    assert "divide" in err(lib)
    for w, s in [(14, 2), (12, 4), (12, 3), (18, 9), (28, 7)]:
        folded = 2 * w ** 4 * 4
        assert lib.wbmm_forward_hier_workspace_bytes(1, 2, 28, 28, w, s, 0, 0, 0) >= folded, (w, s)
        assert lib.wbmm_backward_hier_workspace_bytes(1, 2, 28, 28, w, s, 0, 1) >= folded, (w, s)
        assert hier_fwd(lib, w=w, s=s) == R.WBMM_E_WORKSPACE, (w, s)
        assert hier_bwd(lib, w=w, s=s) == R.WBMM_E_WORKSPACE, (w, s)
    assert hier_fwd(lib, Ts=None) == R.WBMM_E_INVALID
    assert hier_fwd(lib, T=None) == R.WBMM_E_INVALID
    assert hier_fwd(lib, y=FAKE) == R.WBMM_E_INVALID             # y aliases x
    assert hier_fwd(lib, y=0x300000) == R.WBMM_E_INVALID         # y overlaps T_sub
    assert hier_bwd(lib, Ts=None) == R.WBMM_E_INVALID
    assert hier_bwd(lib, mix=0x900000) == R.WBMM_E_INVALID       # mix without z_saved
    assert hier_bwd(lib, dTs=0x300000) == R.WBMM_E_INVALID       # dT_sub aliases T_sub
    assert hier_bwd(lib, dTs=0x500000) == R.WBMM_E_INVALID       # dT_sub aliases dT
    need = lib.wbmm_backward_hier_workspace_bytes(1, 2, 28, 28, 14, 7, 0, 0)
    plain = lib.wbmm_backward_workspace_bytes(1, 2, 28, 28, 14, 0, 0)
    assert need > 0 and plain > 0
    assert hier_bwd(lib) == R.WBMM_E_WORKSPACE
    assert hier_bwd(lib, ws=0xA00000, wsb=need - 1) == R.WBMM_E_WORKSPACE
    assert lib.wbmm_forward_hier_workspace_bytes(1, 2, 128, 128, 14, 7, 0, 1, 0) > 0  # window-mode mix


def test_shifted_validation(lib):
    """Window-grid offsets must lie in [0, w); the rest is checked as in the plain calls."""
    for oy, ox in [(-1, 0), (0, 14), (14, 3), (2, -3)]:
        assert lib.wbmm_forward_shifted(2, 3, 28, 28, 14, oy, ox, 0, 0, 0, FAKE, 0x300000, None,
                                        None, None, FAKE2, None, 0, None) == R.WBMM_E_INVALID
        assert lib.wbmm_backward_shifted(2, 3, 28, 28, 14, oy, ox, 0, FAKE, 0x300000, None, None,
                                         None, 0x400000, FAKE2, None, None, None, 0,
                                         None) == R.WBMM_E_INVALID
        assert lib.wbmm_forward_shifted_workspace_bytes(2, 3, 28, 28, 14, oy, ox, 0, 1, 0) == 0
        assert lib.wbmm_backward_shifted_workspace_bytes(2, 3, 28, 28, 14, oy, ox, 0, 0) == 0
    assert "grid offset" in err(lib)
    # y aliasing x is still caught with a valid offset; the wide-window backward (w = 20) takes
    # offsets too, and needs a workspace
    assert lib.wbmm_forward_shifted(2, 3, 28, 28, 14, 7, 7, 0, 0, 0, FAKE, 0x300000, None, None,
                                    None, FAKE, None, 0, None) == R.WBMM_E_INVALID
    assert lib.wbmm_backward_shifted(2, 3, 40, 40, 20, 10, 10, 0, FAKE, 0x300000, None, None,
                                     None, 0x400000, FAKE2, None, None, None, 0,
                                     None) == R.WBMM_E_WORKSPACE
    assert lib.wbmm_backward_shifted_workspace_bytes(2, 3, 40, 40, 20, 10, 10, 0, 0) > 0
    assert lib.wbmm_backward_shifted_workspace_bytes(2, 3, 28, 28, 14, 7, 7, 0, 0) > 0


def test_shifted_workspace_covers_the_repacked_maps(lib):
    """w = 14 offset grids on NCHW maps: B=64 at 28x28 with offset (5, 9) has 9 windows per image,
    576 windows = 144 repacked 28x28 images of 2x2 windows. The fp32 forward reads the offset
    grid directly (with the mix and no z_save buffer it needs the image-space z, except on the
    rolled map, which applies the mix on chip); the bf16 forward
    without the mix runs on repacked X and z (bf16: together the bytes of one fp32 repacked map);
    the backward holds repacked G, X and dX, and with the mix the image-space G. Offsets of 0 or
    7 on 28x28 maps run on the rolled map instead: the backward from the table then holds only
    the fp64 table-gradient partials (one row of 27 x 27 per 16 images and channel), and the
    image-space G with the mix; the query also covers a cached matrix (general kernels), so the
    figure is the larger of the two, far below one repacked map."""
    B, C = 64, 192
    rep = 144 * C * 28 * 28 * 4
    img = B * C * 28 * 28 * 4
    for oy, ox in ((5, 9), (7, 7)):
        fwd = lib.wbmm_forward_shifted_workspace_bytes(B, C, 28, 28, 14, oy, ox, 0, 0, 0)
        assert fwd >= rep
        assert lib.wbmm_forward_shifted_workspace_bytes(B, C, 28, 28, 14, oy, ox, 0, 1, 1) < img
    assert lib.wbmm_forward_shifted_workspace_bytes(B, C, 28, 28, 14, 5, 9, 0, 1, 0) >= img
    # the rolled-map forward applies the mix on chip: no image-space z without z_save
    assert lib.wbmm_forward_shifted_workspace_bytes(B, C, 28, 28, 14, 7, 7, 0, 1, 0) < img
    bwd = lib.wbmm_backward_shifted_workspace_bytes(B, C, 28, 28, 14, 5, 9, 0, 0)
    assert bwd >= 3 * rep
    assert lib.wbmm_backward_shifted_workspace_bytes(B, C, 28, 28, 14, 5, 9, 0, 1) >= bwd + img
    # a partial last repacked image: 5 images x 9 windows = 45 windows -> 12 repacked images
    assert lib.wbmm_backward_shifted_workspace_bytes(5, 2, 28, 28, 14, 5, 9, 0, 0) >= \
        3 * 12 * 2 * 28 * 28 * 4
    part = C * (B // 16) * 27 * 27 * 8
    for oy, ox in ((7, 7), (7, 0), (0, 7)):
        rolled = lib.wbmm_backward_shifted_workspace_bytes(B, C, 28, 28, 14, oy, ox, 0, 0)
        assert part <= rolled < rep
        assert lib.wbmm_backward_shifted_workspace_bytes(B, C, 28, 28, 14, oy, ox, 0, 1) >= \
            part + img
    # 17 images: two units of 16
    assert lib.wbmm_backward_shifted_workspace_bytes(17, 2, 28, 28, 14, 7, 7, 0, 0) >= \
        2 * 2 * 27 * 27 * 8


def test_backward_bf16_validation(lib):
    """bf16 backward: 1 <= w <= 32 (any layout and map size), mix and z_saved together, workspace
    needed (the fast w = 14 NCHW 28² / 56² shapes, the general and the wide-window ones have
    their own layouts)."""
    def call(B=2, C=3, H=28, W=28, w=14, layout=0, mix=None, z=None, dx=0x500000, ws=0x900000,
             wsb=1 << 30):
        return lib.wbmm_backward_bf16(B, C, H, W, w, layout, FAKE, 0x300000, mix, z, FAKE2, dx,
                                      0x600000, None, ws, wsb, None)
    assert call(w=33) == R.WBMM_E_INVALID
    assert call(w=0) == R.WBMM_E_INVALID
    for kw in ({"H": 30, "W": 30}, {"w": 7}, {"layout": 1}, {"w": 17}, {"w": 28, "layout": 1}):
        # general and wide-window shapes: workspace sized
        need = lib.wbmm_backward_bf16_workspace_bytes(2, 3, kw.get("H", 28), kw.get("W", 28),
                                                      kw.get("w", 14), kw.get("layout", 0), 0)
        assert need > 0
        assert call(ws=0x900000, wsb=need - 1, **kw) == R.WBMM_E_WORKSPACE
    assert call(mix=0x700000) == R.WBMM_E_INVALID            # mix without z_saved
    assert call(dx=FAKE) == R.WBMM_E_INVALID                  # dx aliases x
    assert call(ws=None) == R.WBMM_E_WORKSPACE
    need = lib.wbmm_backward_bf16_workspace_bytes(2, 3, 28, 28, 14, 0, 1)
    assert need > lib.wbmm_backward_bf16_workspace_bytes(2, 3, 28, 28, 14, 0, 0) > 0
    assert call(mix=0x700000, z=0x800000, wsb=need - 1) == R.WBMM_E_WORKSPACE
    assert lib.wbmm_backward_bf16_workspace_bytes(2, 3, 30, 30, 17, 0, 0) > 0
    assert lib.wbmm_backward_bf16_workspace_bytes(2, 3, 30, 30, 33, 0, 0) == 0


def test_probe_validation(lib):
    assert lib.wbmm_probe_mfma(7, 4, 10, FAKE, None) == R.WBMM_E_INVALID
    assert lib.wbmm_probe_mfma(0, 0, 10, FAKE, None) == R.WBMM_E_INVALID
    assert lib.wbmm_probe_mfma(0, 4, 0, FAKE, None) == R.WBMM_E_INVALID
    assert lib.wbmm_probe_mfma(0, 4, 10, None, None) == R.WBMM_E_INVALID
    # flops: blocks x 4 waves x iters x 8 chains x (2*16*16*K), K = 4 (fp32) or 32 (bf16)
    assert lib.wbmm_probe_mfma_flops(0, 3, 5) == 3 * 4 * 5 * 8 * 2048
    assert lib.wbmm_probe_mfma_flops(1, 3, 5) == 3 * 4 * 128 * 8 * 16384   # whole rounds of 128
    assert lib.wbmm_probe_mfma_flops(1, 3, 256) == 3 * 4 * 256 * 8 * 16384
    assert lib.wbmm_probe_mfma_flops(0, 0, 5) == 0.0


def test_dwconv_validation(lib):
    """The DW-Std comparison kernel: odd k in 3..13, rows it can stage, non-overlapping output;
    all rejected on the host."""
    def call(B=2, C=3, H=56, W=56, k=5, x=FAKE, w=0x300000, y=FAKE2):
        return lib.wbmm_dwconv_forward(B, C, H, W, k, x, w, y, None)
    assert call(k=4) == R.WBMM_E_INVALID
    assert call(k=0) == R.WBMM_E_INVALID
    assert call(k=1) == R.WBMM_E_UNSUPPORTED
    assert call(k=15) == R.WBMM_E_UNSUPPORTED
    assert "odd k in 3..13" in err(lib)
    assert call(W=1100) == R.WBMM_E_UNSUPPORTED          # a row too long to stage
    assert call(B=0) == R.WBMM_E_INVALID
    assert call(x=None) == R.WBMM_E_INVALID
    assert call(w=None) == R.WBMM_E_INVALID
    assert call(y=FAKE) == R.WBMM_E_INVALID              # y aliases x
    assert call(y=0x300000) == R.WBMM_E_INVALID          # y overlaps the weights
    assert call(x=FAKE + 2) == R.WBMM_E_UNSUPPORTED      # misaligned


def test_last_error_is_per_thread(lib):
    import threading
    assert lib.wbmm_build_index(0, FAKE, None) == R.WBMM_E_INVALID
    seen = []
    t = threading.Thread(target=lambda: seen.append(lib.wbmm_last_error()))
    t.start()
    t.join()
    assert seen == [b""]
    assert err(lib) != ""


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(R.WbmmError):
        R.load_library(str(tmp_path / "nope.so"))
    R.load_library()  # restore
