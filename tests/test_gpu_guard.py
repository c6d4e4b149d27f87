"""Guard bands: every output (and the workspace) of every kernel path is placed inside a larger
buffer whose margins hold a sentinel bit pattern; after the call the margins must be untouched.

A store past either end of an output (for instance a part-empty last unit, or tiles of images
past the batch) would otherwise land in unrelated memory unseen. Batches are ragged so that the
last unit of each fast kernel is part empty. The outputs are also checked against the oracle.
"""
import numpy as np
import pytest

from oracle import wbmm_oracle as O
from receptive_field_spatial_amd import synth
from tests.parity_util import assert_bf16, assert_f32

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

GUARD_BYTES = 64 * 1024        # each margin; a multiple of 256 so the output stays aligned
SENT32 = 0x7FC0DEAD            # a NaN no kernel writes
SENT16 = 0x7FAD                # a bf16 NaN pattern


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import receptive_field_spatial_amd as R
    R.load_library()


def R():
    import receptive_field_spatial_amd as mod
    return mod


def say(msg):
    print(f"\n[case] {msg}", flush=True)


class Guarded:
    """A tensor of `shape`/`dtype` inside a buffer with sentinel margins on both sides."""

    def __init__(self, shape, dtype=torch.float32):
        self.shape = tuple(shape)
        self.dtype = dtype
        esz = torch.empty((), dtype=dtype).element_size()
        n = int(np.prod(self.shape)) if self.shape else 1
        self.g = GUARD_BYTES // esz
        self.n = n
        if esz == 4:
            self.fill, bdt = SENT32, torch.int32
        elif esz == 2:
            self.fill, bdt = SENT16, torch.int16
        else:  # bytes (workspaces)
            self.fill, bdt = 0xA5 - 256, torch.int8
        self.buf = torch.full((n + 2 * self.g,), self.fill, dtype=bdt, device="cuda")
        self.t = self.buf[self.g:self.g + n].view(dtype).view(self.shape)

    def check(self, what):
        torch.cuda.synchronize()
        head = self.buf[:self.g]
        tail = self.buf[self.g + self.n:]
        bad_h = int((head != self.fill).sum())
        bad_t = int((tail != self.fill).sum())
        assert bad_h == 0 and bad_t == 0, f"{what}: {bad_h} elements before, {bad_t} after written"


def dev(a, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype).cuda()


def dev_bf16(a_f32):
    bits = synth.f32_to_bf16_bits(a_f32).view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.bfloat16).cuda()


def host(t):
    return t.float().cpu().numpy()


def guarded_ws(nbytes):
    return Guarded((max(int(nbytes), 1),), torch.uint8) if nbytes else None


# fp32 fast shapes (w = 14 on 14², 28², 56² NCHW) with ragged batches, plus general-kernel cases
F32_CASES = [(5, 3, 14, 14, 14), (17, 3, 28, 28, 14), (3, 2, 56, 56, 14), (5, 2, 56, 56, 14),
             (2, 3, 30, 25, 14), (3, 2, 10, 13, 4), (1, 2, 100, 100, 14)]


@pytest.mark.parametrize("B,C,H,W,w", F32_CASES)
@pytest.mark.parametrize("mix", [False, True])
def test_guard_fp32_layer(B, C, H, W, w, mix):
    """Forward (y, z_save, workspace) and backward (dx, dT, dWmix, workspace) in guarded
    buffers."""
    say(f"guard fp32 B={B} C={C} H={H} W={W} w={w} mix={mix}")
    x = synth.normal_f32((B, C, H, W), 1.0, seed=400)
    T = synth.normal_f32((C, 2 * w - 1, 2 * w - 1), 0.02, seed=401)
    Wm = synth.normal_f32((C, 3, 3), 0.1, seed=402) if mix else None
    dy = synth.normal_f32((B, C, H, W), 1.0, seed=403)
    xd, Td, dyd = dev(x), dev(T), dev(dy)
    Wd = dev(Wm) if mix else None
    y, z = Guarded(x.shape), Guarded(x.shape)
    wsf = guarded_ws(R().wbmm_forward_workspace_bytes(B, C, H, W, w, has_mix=mix,
                                                      has_z_save=True))
    R().wbmm_forward(xd, w, T=Td, mix_w=Wd, y=y.t, z_save=z.t,
                     workspace=wsf.t if wsf else None)
    y.check("y")
    z.check("z_save")
    if wsf:
        wsf.check("forward workspace")
    L = 2 * w - 1
    dx, dT = Guarded(x.shape), Guarded((C, L, L))
    dW = Guarded((C, 3, 3)) if mix else None
    wsb = guarded_ws(R().wbmm_backward_workspace_bytes(B, C, H, W, w, has_mix=mix))
    R().wbmm_backward(xd, dyd, w, T=Td, mix_w=Wd, z_saved=z.t if mix else None, dx=dx.t, dT=dT.t,
                      dmix_w=dW.t if mix else False, workspace=wsb.t if wsb else None)
    dx.check("dx")
    dT.check("dT")
    if mix:
        dW.check("dWmix")
    if wsb:
        wsb.check("backward workspace")
    wy, wz = O.layer_forward(x.astype(np.float64), w, T=T, Wmix=Wm)
    assert_f32(host(y.t), wy, "y")
    assert_f32(host(z.t), wz, "z")
    wdx, wdT, wdW = O.layer_backward(x.astype(np.float64), dy.astype(np.float64), w, T=T, Wmix=Wm,
                                     z=host(z.t).astype(np.float64) if mix else None)
    assert_f32(host(dx.t), wdx, "dx")
    assert_f32(host(dT.t), wdT, "dT")
    if mix:
        assert_f32(host(dW.t), wdW, "dWmix")


# forward-only fast fp32 kernels: w = 7 and w = 28 on 56x56 maps (ragged batches against the
# w = 28 kernel's 8-image blocks), and the cached-matrix kernel (whole and border windows)
F32_FWD_CASES = [(5, 2, 56, 56, 7, False), (9, 2, 56, 56, 28, False), (3, 2, 56, 56, 28, False),
                 (5, 3, 56, 56, 14, True), (3, 3, 28, 28, 14, True), (2, 2, 100, 100, 14, True),
                 (2, 3, 100, 100, 14, False), (3, 2, 30, 44, 14, False)]


@pytest.mark.parametrize("B,C,H,W,w,cached", F32_FWD_CASES)
@pytest.mark.parametrize("mix", [False, True])
def test_guard_fp32_forward_fast(B, C, H, W, w, cached, mix):
    """y, z_save and the workspace of the forward-only fast kernels in guarded buffers."""
    say(f"guard fp32 forward B={B} C={C} H={H} W={W} w={w} cached={cached} mix={mix}")
    x = synth.normal_f32((B, C, H, W), 1.0, seed=410)
    T = synth.normal_f32((C, 2 * w - 1, 2 * w - 1), 0.02, seed=411)
    Wm = synth.normal_f32((C, 3, 3), 0.1, seed=412) if mix else None
    xd, Td = dev(x), dev(T)
    kw = {"M": R().wbmm_build_matrix(Td, w)} if cached else {"T": Td}
    for zsave in (False, True):
        y = Guarded(x.shape)
        z = Guarded(x.shape) if zsave else None
        wsf = guarded_ws(R().wbmm_forward_workspace_bytes(B, C, H, W, w, has_mix=mix,
                                                          has_z_save=zsave))
        R().wbmm_forward(xd, w, mix_w=dev(Wm) if mix else None, y=y.t,
                         z_save=z.t if zsave else None, workspace=wsf.t if wsf else None, **kw)
        y.check("y")
        if zsave:
            z.check("z_save")
        if wsf:
            wsf.check("forward workspace")
        wy, wz = O.layer_forward(x.astype(np.float64), w, T=T, Wmix=Wm)
        assert_f32(host(y.t), wy, "y")
        if zsave:
            assert_f32(host(z.t), wz, "z")


@pytest.mark.parametrize("B,C,H", [(5, 3, 14), (18, 2, 28), (5, 2, 56), (2, 3, 30)])
@pytest.mark.parametrize("mix", [False, True])
def test_guard_hier(B, C, H, mix):
    """The kernels with the fold on chip (whole images; a padded map: the table kernel forward,
    the general backward): y, z_save, dx, dT, dT_sub, dWmix guarded."""
    w, s = 14, 7
    say(f"guard hier B={B} C={C} H=W={H} mix={mix}")
    x = synth.normal_f32((B, C, H, H), 1.0, seed=410)
    T = synth.normal_f32((C, 27, 27), 0.02, seed=411)
    Ts = synth.normal_f32((C, 13, 13), 0.02, seed=412)
    Wm = synth.normal_f32((C, 3, 3), 0.1, seed=413) if mix else None
    dy = synth.normal_f32((B, C, H, H), 1.0, seed=414)
    xd, Td, Tsd, dyd = dev(x), dev(T), dev(Ts), dev(dy)
    Wd = dev(Wm) if mix else None
    y, z = Guarded(x.shape), Guarded(x.shape)
    R().wbmm_forward_hier(xd, w, s, Td, Tsd, mix_w=Wd, y=y.t, z_save=z.t)
    y.check("y")
    z.check("z_save")
    dx, dT, dTs = Guarded(x.shape), Guarded((C, 27, 27)), Guarded((C, 13, 13))
    dW = Guarded((C, 3, 3)) if mix else None
    wsb = guarded_ws(R().wbmm_backward_hier_workspace_bytes(B, C, H, H, w, s, has_mix=mix))
    R().wbmm_backward_hier(xd, dyd, w, s, Td, Tsd, mix_w=Wd, z_saved=z.t if mix else None,
                           dx=dx.t, dT=dT.t, dT_sub=dTs.t, dmix_w=dW.t if mix else False,
                           workspace=wsb.t if wsb else None)
    for g, n in ((dx, "dx"), (dT, "dT"), (dTs, "dT_sub")):
        g.check(n)
    if mix:
        dW.check("dWmix")
    if wsb:
        wsb.check("backward workspace")
    wy, wz = O.layer_forward_hier(x.astype(np.float64), w, s, T, Ts, Wmix=Wm)
    assert_f32(host(y.t), wy, "y")
    wdx, wdT, wdTs, wdW = O.layer_backward_hier(x.astype(np.float64), dy.astype(np.float64), w, s,
                                                T, Ts, Wmix=Wm,
                                                z=host(z.t).astype(np.float64) if mix else None)
    assert_f32(host(dx.t), wdx, "dx")
    assert_f32(host(dT.t), wdT, "dT")
    assert_f32(host(dTs.t), wdTs, "dT_sub")


@pytest.mark.parametrize("B,C,H,W,w,s", [(2, 3, 24, 24, 12, 4), (1, 2, 26, 20, 12, 3),
                                         (1, 2, 36, 36, 18, 9)])
@pytest.mark.parametrize("mix", [False, True])
def test_guard_hier_general(B, C, H, W, w, s, mix):
    """The fold for s other than w / 2 (and w = 2s above 16) goes through a folded matrix in the
    workspace: y, z_save, both workspaces, dx, dT, dT_sub and dWmix guarded."""
    say(f"guard hier general B={B} C={C} H={H} W={W} w={w} s={s} mix={mix}")
    L1, Ls = 2 * w - 1, 2 * s - 1
    x = synth.normal_f32((B, C, H, W), 1.0, seed=420)
    T = synth.normal_f32((C, L1, L1), 0.02, seed=421)
    Ts = synth.normal_f32((C, Ls, Ls), 0.02, seed=422)
    Wm = synth.normal_f32((C, 3, 3), 0.1, seed=423) if mix else None
    dy = synth.normal_f32((B, C, H, W), 1.0, seed=424)
    xd, Td, Tsd, dyd = dev(x), dev(T), dev(Ts), dev(dy)
    Wd = dev(Wm) if mix else None
    y, z = Guarded(x.shape), Guarded(x.shape)
    wsf = guarded_ws(R().wbmm_forward_hier_workspace_bytes(B, C, H, W, w, s, has_mix=mix,
                                                            has_z_save=True))
    assert wsf is not None
    R().wbmm_forward_hier(xd, w, s, Td, Tsd, mix_w=Wd, y=y.t, z_save=z.t, workspace=wsf.t)
    y.check("y")
    z.check("z_save")
    wsf.check("forward workspace")
    dx, dT, dTs = Guarded(x.shape), Guarded((C, L1, L1)), Guarded((C, Ls, Ls))
    dW = Guarded((C, 3, 3)) if mix else None
    wsb = guarded_ws(R().wbmm_backward_hier_workspace_bytes(B, C, H, W, w, s, has_mix=mix))
    assert wsb is not None
    R().wbmm_backward_hier(xd, dyd, w, s, Td, Tsd, mix_w=Wd, z_saved=z.t if mix else None,
                           dx=dx.t, dT=dT.t, dT_sub=dTs.t, dmix_w=dW.t if mix else False,
                           workspace=wsb.t)
    for g, n in ((dx, "dx"), (dT, "dT"), (dTs, "dT_sub")):
        g.check(n)
    if mix:
        dW.check("dWmix")
    wsb.check("backward workspace")
    wy, _ = O.layer_forward_hier(x.astype(np.float64), w, s, T, Ts, Wmix=Wm)
    assert_f32(host(y.t), wy, "y")
    wdx, wdT, wdTs, wdW = O.layer_backward_hier(x.astype(np.float64), dy.astype(np.float64), w, s,
                                                T, Ts, Wmix=Wm,
                                                z=host(z.t).astype(np.float64) if mix else None)
    assert_f32(host(dx.t), wdx, "dx")
    assert_f32(host(dT.t), wdT, "dT")
    assert_f32(host(dTs.t), wdTs, "dT_sub")
    if mix:
        assert_f32(host(dW.t), wdW, "dWmix")


@pytest.mark.parametrize("w,hw,B", [(14, 28, 5), (14, 56, 3), (7, 56, 5), (28, 56, 3),
                                    (28, 56, 21), (14, 14, 3)])
@pytest.mark.parametrize("mix", [False, True])
def test_guard_bf16_forward(w, hw, B, mix):
    """bf16 forwards (the fast w = 7/14/28 kernels, whose tiles of images past the batch are
    clamped to the last image): y and z_save guarded."""
    C = 3
    say(f"guard bf16 forward w={w} {hw}x{hw} B={B} mix={mix}")
    x = synth.round_to_bf16(synth.normal_f32((B, C, hw, hw), 1.0, seed=420))
    T = synth.round_to_bf16(synth.normal_f32((C, 2 * w - 1, 2 * w - 1), 0.02, seed=421))
    Wm = synth.normal_f32((C, 3, 3), 0.1, seed=422) if mix else None
    y, z = Guarded(x.shape, torch.bfloat16), Guarded(x.shape, torch.bfloat16)
    wsf = guarded_ws(R().wbmm_forward_workspace_bytes(B, C, hw, hw, w, has_mix=mix,
                                                      has_z_save=True))
    R().wbmm_forward(dev_bf16(x), w, T=dev_bf16(T), mix_w=dev(Wm) if mix else None,
                     out_dtype=torch.bfloat16, y=y.t, z_save=z.t,
                     workspace=wsf.t if wsf else None)
    y.check("y")
    z.check("z_save")
    if wsf:
        wsf.check("forward workspace")
    wy, wz = O.layer_forward(x.astype(np.float64), w, T=T, Wmix=Wm)
    assert_bf16(host(y.t), wy, "y")
    assert_bf16(host(z.t), wz, "z")


@pytest.mark.parametrize("B,H", [(5, 28), (3, 56)])
@pytest.mark.parametrize("mix", [False, True])
def test_guard_bf16_backward(B, H, mix):
    """bf16 backward: dx (bf16), dT, dWmix and the workspace guarded."""
    w, C = 14, 3
    say(f"guard bf16 backward B={B} H=W={H} mix={mix}")
    x = synth.round_to_bf16(synth.normal_f32((B, C, H, H), 1.0, seed=430))
    T = synth.round_to_bf16(synth.normal_f32((C, 27, 27), 0.02, seed=431))
    dy = synth.round_to_bf16(synth.normal_f32((B, C, H, H), 1.0, seed=432))
    Wm = synth.normal_f32((C, 3, 3), 0.1, seed=433) if mix else None
    z = (synth.round_to_bf16(O.wbmm_forward(x.astype(np.float64), w, T=T).astype(np.float32))
         if mix else None)
    dx, dT = Guarded(x.shape, torch.bfloat16), Guarded((C, 27, 27))
    dW = Guarded((C, 3, 3)) if mix else None
    wsb = guarded_ws(R().wbmm_backward_bf16_workspace_bytes(B, C, H, H, w, has_mix=mix))
    R().wbmm_backward_bf16(dev_bf16(x), dev_bf16(dy), w, dev_bf16(T),
                           mix_w=dev(Wm) if mix else None, z_saved=dev_bf16(z) if mix else None,
                           dx=dx.t, dT=dT.t, dmix_w=dW.t if mix else False, workspace=wsb.t)
    dx.check("dx")
    dT.check("dT")
    if mix:
        dW.check("dWmix")
    wsb.check("backward workspace")
    wdx, wdT, wdW = O.layer_backward(x.astype(np.float64), dy.astype(np.float64), w, T=T, Wmix=Wm,
                                     z=z.astype(np.float64) if mix else None)
    assert_bf16(host(dx.t), wdx, "dx")
    assert_bf16(host(dT.t), wdT, "dT")


@pytest.mark.parametrize("B,C,H,W,w,o", [(5, 3, 28, 28, 14, 7), (2, 2, 30, 25, 14, 3),
                                         (2, 2, 17, 13, 4, 2), (17, 3, 28, 28, 14, 7),
                                         (3, 2, 56, 56, 14, 7), (66, 2, 14, 14, 14, 7)])
def test_guard_shifted(B, C, H, W, w, o):
    """The interleaved grid (the rolled-map kernels for offset 7 on 28x28 maps, the table kernel
    and repacked fast kernels for other w = 14 grids): outputs and workspaces guarded."""
    say(f"guard shifted B={B} C={C} H={H} W={W} w={w} o={o}")
    x = synth.normal_f32((B, C, H, W), 1.0, seed=440)
    T = synth.normal_f32((C, 2 * w - 1, 2 * w - 1), 0.05, seed=441)
    Wm = synth.normal_f32((C, 3, 3), 0.1, seed=442)
    dy = synth.normal_f32((B, C, H, W), 1.0, seed=443)
    xd, Td, Wd, dyd = dev(x), dev(T), dev(Wm), dev(dy)
    y, z = Guarded(x.shape), Guarded(x.shape)
    wsf = guarded_ws(R().wbmm_forward_shifted_workspace_bytes(B, C, H, W, w, o, o, has_mix=True,
                                                              has_z_save=True))
    R().wbmm_forward_shifted(xd, w, o, o, T=Td, mix_w=Wd, y=y.t, z_save=z.t,
                             workspace=wsf.t if wsf else None)
    y.check("y")
    z.check("z_save")
    if wsf:
        wsf.check("forward workspace")
    L = 2 * w - 1
    dx, dT, dW = Guarded(x.shape), Guarded((C, L, L)), Guarded((C, 3, 3))
    wsb = guarded_ws(R().wbmm_backward_shifted_workspace_bytes(B, C, H, W, w, o, o, has_mix=True))
    R().wbmm_backward_shifted(xd, dyd, w, o, o, T=Td, mix_w=Wd, z_saved=z.t, dx=dx.t, dT=dT.t,
                              dmix_w=dW.t, workspace=wsb.t if wsb else None)
    for g, n in ((dx, "dx"), (dT, "dT"), (dW, "dWmix")):
        g.check(n)
    if wsb:
        wsb.check("backward workspace")
    wy, _ = O.layer_forward_shifted(x.astype(np.float64), w, o, o, T=T, Wmix=Wm)
    assert_f32(host(y.t), wy, "y")
    wdx, wdT, wdW = O.layer_backward_shifted(x.astype(np.float64), dy.astype(np.float64), w, o, o,
                                             T=T, Wmix=Wm, z=host(z.t).astype(np.float64))
    assert_f32(host(dx.t), wdx, "dx")
    assert_f32(host(dT.t), wdT, "dT")
    assert_f32(host(dW.t), wdW, "dWmix")


@pytest.mark.parametrize("k,B,C,H,W", [(5, 2, 3, 56, 56), (13, 1, 2, 13, 17), (7, 3, 2, 28, 28)])
def test_guard_dwconv(k, B, C, H, W):
    say(f"guard dwconv k={k} B={B} C={C} H={H} W={W}")
    x = synth.normal_f32((B, C, H, W), 1.0, seed=450)
    Wd = synth.normal_f32((C, k, k), 0.05, seed=451)
    y = Guarded(x.shape)
    R().wbmm_dwconv_forward(dev(x), dev(Wd), y=y.t)
    y.check("y")
    assert_f32(host(y.t), O.dw_conv_forward(x.astype(np.float64), Wd), "y")


@pytest.mark.parametrize("w,s,C", [(14, 7, 3), (28, 7, 1), (4, 2, 2)])
def test_guard_index_matrix_fold(w, s, C):
    """idx, M and the folded M' in guarded buffers (bitwise against the oracle)."""
    say(f"guard index/matrix/fold w={w} s={s} C={C}")
    d = w * w
    idx = Guarded((d, d), torch.int32)
    R().wbmm_build_index(w, out=idx.t)
    idx.check("idx")
    assert np.array_equal(idx.t.cpu().numpy(), O.build_index(w))
    T = synth.normal_f32((C, 2 * w - 1, 2 * w - 1), 0.02, seed=460)
    Ts = synth.normal_f32((C, 2 * s - 1, 2 * s - 1), 0.02, seed=461)
    M = Guarded((C, d, d))
    R().wbmm_build_matrix(dev(T), w, out=M.t)
    M.check("M")
    Mf = Guarded((C, d, d))
    R().wbmm_fold_hier(M.t, dev(Ts), w, s, out=Mf.t)
    Mf.check("M'")
    assert np.array_equal(host(Mf.t), O.fold_hier(O.build_matrix(T, w), Ts, w, s))
