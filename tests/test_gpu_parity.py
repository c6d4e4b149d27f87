"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, element by element.

Every case prints its name, shapes and seed before touching the GPU. Inputs come from the seeded
generators in receptive_field_spatial_amd.synth; expected values come only from oracle/.
"""
import numpy as np
import pytest

from oracle import wbmm_oracle as O
from receptive_field_spatial_amd import synth
from tests.parity_util import assert_bf16, assert_f32

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import receptive_field_spatial_amd as R
    R.load_library()
    return R


def R():
    import receptive_field_spatial_amd as mod
    return mod


def say(msg):
    print(f"\n[case] {msg}", flush=True)


def dev(a, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype).cuda()


def dev_bf16(a_f32):
    """bf16-valued float32 numpy -> torch bfloat16 on the GPU (exact)."""
    bits = synth.f32_to_bf16_bits(a_f32).view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.bfloat16).cuda()


def host(t):
    return t.float().cpu().numpy()


# ----------------------------------------------------------------------------- index / matrix
@pytest.mark.parametrize("w", [1, 2, 3, 5, 7, 14, 16, 28, 32])
def test_build_index_bit_exact(w):
    say(f"build_index w={w}")
    got = R().wbmm_build_index(w)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), O.build_index(w))


@pytest.mark.parametrize("w,C", [(1, 2), (4, 3), (7, 8), (14, 5), (28, 2)])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_build_matrix_bit_exact(w, C, dt):
    say(f"build_matrix w={w} C={C} {dt}")
    T = synth.normal_f32((C, 2 * w - 1, 2 * w - 1), 0.02, seed=w)
    if dt == "bf16":
        T = synth.round_to_bf16(T)
        got = R().wbmm_build_matrix(dev_bf16(T), w)
    else:
        got = R().wbmm_build_matrix(dev(T), w)
    want = O.build_matrix(T, w)
    assert np.array_equal(host(got), want)


@pytest.mark.parametrize("w,s,C", [(14, 7, 4), (4, 2, 3), (6, 3, 2), (12, 4, 2), (28, 7, 1)])
def test_fold_bit_exact_f32(w, s, C):
    say(f"fold_hier f32 w={w} s={s} C={C}")
    T = synth.normal_f32((C, 2 * w - 1, 2 * w - 1), 0.02, seed=1)
    Ts = synth.normal_f32((C, 2 * s - 1, 2 * s - 1), 0.02, seed=2)
    M = R().wbmm_build_matrix(dev(T), w)
    got = R().wbmm_fold_hier(M, dev(Ts), w, s)
    want = O.fold_hier(O.build_matrix(T, w), Ts, w, s)
    assert np.array_equal(host(got), want)
    # in place
    R().wbmm_fold_hier(M, dev(Ts), w, s, out=M)
    assert np.array_equal(host(M), want)


def test_fold_bf16_rounds_once():
    w, s, C = 14, 7, 2
    say("fold_hier bf16 w=14 s=7")
    T = synth.round_to_bf16(synth.normal_f32((C, 27, 27), 0.02, seed=3))
    Ts = synth.round_to_bf16(synth.normal_f32((C, 13, 13), 0.02, seed=4))
    got = R().wbmm_fold_hier(R().wbmm_build_matrix(dev_bf16(T), w), dev_bf16(Ts), w, s)
    # oracle: fp32 add of the two bf16 values, then one RNE rounding to bf16
    want = synth.round_to_bf16(O.fold_hier(O.build_matrix(T, w), Ts, w, s))
    assert np.array_equal(host(got), want)


# ----------------------------------------------------------------------------- forward fp32
def fwd_case(B, C, H, W, w, *, cached=False, mix=False, layout="NCHW", seed=0, zsave=False):
    x = synth.normal_f32((B, C, H, W), 1.0, seed=seed)
    T = synth.normal_f32((C, 2 * w - 1, 2 * w - 1), 0.02, seed=seed + 1)
    Wm = synth.normal_f32((C, 3, 3), 0.1, seed=seed + 2) if mix else None
    xd = dev(x if layout == "NCHW" else x.transpose(0, 2, 3, 1))
    Td = dev(T)
    kw = {}
    if cached:
        kw["M"] = R().wbmm_build_matrix(Td, w)
    else:
        kw["T"] = Td
    zs = torch.empty_like(xd) if zsave else None
    y = R().wbmm_forward(xd, w, mix_w=dev(Wm) if mix else None, layout=layout, z_save=zs, **kw)
    yh = host(y)
    zh = host(zs) if zsave else None
    if layout == "NHWC":
        yh = yh.transpose(0, 3, 1, 2)
        zh = zh.transpose(0, 3, 1, 2) if zsave else None
    want_y, want_z = O.layer_forward(x.astype(np.float64), w, T=T.astype(np.float64), Wmix=Wm)
    return yh, want_y, zh, want_z


@pytest.mark.parametrize("cached", [False, True])
def test_forward_tiny_workload(cached):
    wl = synth.WORKLOADS["tiny_w7"]
    say(f"forward tiny_w7 cached={cached}")
    inp = synth.draw_inputs(wl)
    x, T = inp["x"], inp["T"]
    kw = {"M": R().wbmm_build_matrix(dev(T), wl.w)} if cached else {"T": dev(T)}
    y = R().wbmm_forward(dev(x), wl.w, **kw)
    assert_f32(host(y), O.wbmm_forward(x.astype(np.float64), wl.w, T=T.astype(np.float64)), "y")


@pytest.mark.parametrize("B,C,H,W,w", [
    (2, 3, 10, 13, 4),    # padding on both axes
    (1, 2, 5, 5, 5),      # one window
    (3, 2, 7, 3, 3),      # tall/narrow ragged
    (2, 2, 4, 4, 1),      # w = 1
    (2, 3, 30, 17, 6),
    (1, 2, 33, 47, 8),
    (2, 2, 20, 21, 10),
    (1, 3, 28, 42, 14),
    (5, 3, 14, 14, 14),   # fast 14x14 kernel: one unit of 64 images, part empty
    (3, 2, 56, 56, 14),   # fast 56x56 kernel: last unit part empty
    (2, 2, 30, 30, 15),
    (1, 2, 32, 48, 16),
    (1, 2, 40, 37, 20),   # w > 16: rows split over waves
    (1, 1, 56, 56, 28),
    (1, 1, 40, 64, 32),
])
@pytest.mark.parametrize("cached", [False, True])
def test_forward_shapes(B, C, H, W, w, cached):
    say(f"forward shapes B={B} C={C} H={H} W={W} w={w} cached={cached}")
    yh, want, _, _ = fwd_case(B, C, H, W, w, cached=cached)
    assert_f32(yh, want, "y")


@pytest.mark.parametrize("B,C", [(1, 3), (5, 2), (16, 2), (17, 3), (33, 2)])
@pytest.mark.parametrize("mix", [False, True])
@pytest.mark.parametrize("zsave", [False, True])
def test_forward_f32_28x28_w14(B, C, mix, zsave):
    """fp32 w = 14 on 28x28 NCHW images (the training shape's own forward kernel): ragged batches
    (images past the batch are clamped), with and without the fused mix and z_save."""
    say(f"forward f32 28x28 w=14 B={B} C={C} mix={mix} zsave={zsave}")
    yh, want_y, zh, want_z = fwd_case(B, C, 28, 28, 14, cached=False, mix=mix, zsave=zsave)
    assert_f32(yh, want_y, "y")
    if zsave:
        assert_f32(zh, want_z, "z")


@pytest.mark.parametrize("B,C,mix", [(16, 600, False), (5, 300, False), (16, 600, True),
                                     (64, 1800, True), (37, 1000, True)])
def test_forward_f32_28x28_w14_shift_bitwise(B, C, mix):
    """One-hot tables at a different offset in every channel (fp32, 28x28, w = 14): the output is
    the input shifted inside each window, bit for bit. More units than resident workgroups, so
    workgroups walk several units and restage the table when the channel changes. With `mix`,
    the mix weights are the identity (one-hot centre) and z_save is taken: both y and z_save are
    the shifted input, bit for bit, which checks the mix sweep's addressing over many units."""
    w = 14
    say(f"forward f32 28x28 shift B={B} C={C} mix={mix}")
    x = synth.normal_f32((B, C, 28, 28), 1.0, seed=35)
    dy = (np.arange(C) * 5) % 27 - 13
    dx = (np.arange(C) * 11 + 3) % 27 - 13
    T = np.zeros((C, 27, 27), np.float32)
    T[np.arange(C), dy + 13, dx + 13] = 1.0
    want = _window_shift(x, w, dy, dx)
    if not mix:
        y = R().wbmm_forward(dev(x), w, T=dev(T))
        assert np.array_equal(host(y), want)
        return
    W9 = np.zeros((C, 3, 3), np.float32)
    W9[:, 1, 1] = 1.0
    xd = dev(x)
    z = torch.empty_like(xd)
    y = R().wbmm_forward(xd, w, T=dev(T), mix_w=dev(W9), z_save=z)
    assert np.array_equal(host(z), want)
    assert np.array_equal(host(y), want)


@pytest.mark.parametrize("hw,B,C,mix", [(56, 4, 700, False), (56, 5, 300, True),
                                         (56, 13, 256, True), (14, 70, 600, True),
                                         (14, 64, 300, False)])
def test_forward_f32_w14_shift_bitwise_all_channels(hw, B, C, mix):
    """As the 28x28 case, on the fast fp32 kernels for 56x56 and 14x14 images: one-hot tables at
    a different offset in every channel (and the identity mix with z_save), so that every
    channel's output is the input shifted inside each window, bit for bit. With more units than
    resident workgroups, this checks the units' walk over channels and images at full width."""
    w = 14
    say(f"forward f32 {hw}x{hw} shift all channels B={B} C={C} mix={mix}")
    x = synth.normal_f32((B, C, hw, hw), 1.0, seed=36)
    dy = (np.arange(C) * 7 + 1) % 27 - 13
    dx = (np.arange(C) * 3 + 5) % 27 - 13
    T = np.zeros((C, 27, 27), np.float32)
    T[np.arange(C), dy + 13, dx + 13] = 1.0
    want = _window_shift(x, w, dy, dx)
    xd = dev(x)
    if not mix:
        assert np.array_equal(host(R().wbmm_forward(xd, w, T=dev(T))), want)
        return
    W9 = np.zeros((C, 3, 3), np.float32)
    W9[:, 1, 1] = 1.0
    z = torch.empty_like(xd)
    y = R().wbmm_forward(xd, w, T=dev(T), mix_w=dev(W9), z_save=z)
    assert np.array_equal(host(z), want)
    assert np.array_equal(host(y), want)


@pytest.mark.parametrize("B,C,H,W,w", [(2, 3, 28, 28, 14), (1, 4, 10, 13, 4), (3, 2, 56, 56, 7),
                                       (1, 3, 150, 74, 14)])
@pytest.mark.parametrize("cached", [False, True])
def test_forward_mix_and_zsave(B, C, H, W, w, cached):
    say(f"forward mix+zsave B={B} C={C} H={H} W={W} w={w} cached={cached}")
    yh, want_y, zh, want_z = fwd_case(B, C, H, W, w, cached=cached, mix=True, zsave=True)
    assert_f32(yh, want_y, "y")
    assert_f32(zh, want_z, "z")


def test_forward_mix_window_mode():
    """Images too large for one workgroup (100 windows): the mix runs as its own pass."""
    say("forward mix window mode B=1 C=2 H=W=128 w=14")
    yh, want_y, zh, want_z = fwd_case(1, 2, 128, 128, 14, mix=True, zsave=True)
    assert_f32(yh, want_y, "y")
    assert_f32(zh, want_z, "z")
    yh, want_y, _, _ = fwd_case(1, 2, 128, 128, 14, mix=True, zsave=False)
    assert_f32(yh, want_y, "y (workspace)")


@pytest.mark.parametrize("w", [4, 7, 14])
def test_forward_nhwc(w):
    say(f"forward NHWC w={w}")
    yh, want, _, _ = fwd_case(2, 5, 2 * w + 3, 3 * w - 2, w, layout="NHWC")
    assert_f32(yh, want, "y")
    yh, want, _, _ = fwd_case(2, 5, 28, 28, w, layout="NHWC", mix=True)
    assert_f32(yh, want, "y mix")


@pytest.mark.parametrize("w", [1, 4, 7, 14, 28])
@pytest.mark.parametrize("cached", [False, True])
def test_forward_one_hot_identity_bitwise(w, cached):
    """Centre one-hot table: products with 0 and 1 are exact, so the output equals x bitwise."""
    say(f"one-hot identity w={w} cached={cached}")
    C = 3
    x = synth.normal_f32((2, C, 2 * w + 1, w + 3), 1.0, seed=5)
    T = np.zeros((C, 2 * w - 1, 2 * w - 1), np.float32)
    T[:, w - 1, w - 1] = 1.0
    kw = {"M": R().wbmm_build_matrix(dev(T), w)} if cached else {"T": dev(T)}
    y = R().wbmm_forward(dev(x), w, **kw)
    assert np.array_equal(host(y), x)


def test_forward_one_hot_shift_bitwise():
    w, C = 7, 2
    say("one-hot shift w=7")
    x = synth.normal_f32((1, C, 14, 21), 1.0, seed=6)
    T = np.zeros((C, 13, 13), np.float32)
    T[:, w - 1 + 2, w - 1 - 1] = 1.0  # out(y, x) = in(y - 2, x + 1)
    y = host(R().wbmm_forward(dev(x), w, T=dev(T)))
    want = O.wbmm_forward(x.astype(np.float64), w, T=T.astype(np.float64))
    assert np.array_equal(y, want.astype(np.float32))


# ----------------------------------------------------------------------------- forward bf16
@pytest.mark.parametrize("w", [4, 7, 14, 28])
@pytest.mark.parametrize("cached", [False, True])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_forward_bf16(w, cached, out):
    say(f"forward bf16 w={w} cached={cached} out={out}")
    B, C, H, W = 2, 3, 2 * w + 5, 2 * w
    x = synth.round_to_bf16(synth.normal_f32((B, C, H, W), 1.0, seed=7))
    T = synth.round_to_bf16(synth.normal_f32((C, 2 * w - 1, 2 * w - 1), 0.02, seed=8))
    Td = dev_bf16(T)
    kw = {"M": R().wbmm_build_matrix(Td, w)} if cached else {"T": Td}
    od = torch.bfloat16 if out == "bf16" else torch.float32
    y = R().wbmm_forward(dev_bf16(x), w, out_dtype=od, **kw)
    want = O.wbmm_forward(x.astype(np.float64), w, T=T.astype(np.float64))
    assert_bf16(host(y), want, "y")
    if out == "f32":  # fp32 output: only accumulation-order differences remain
        assert_f32(host(y), want, "y (fp32 out)")


@pytest.mark.parametrize("w,hw,B", [(14, 14, 3), (14, 28, 5), (14, 28, 16), (14, 28, 33), (14, 56, 3),
                                    (14, 56, 6), (14, 56, 9), (7, 56, 3), (7, 56, 4), (7, 56, 9),
                                    (28, 56, 3), (28, 56, 16), (28, 56, 21)])
@pytest.mark.parametrize("zsave", [False, True])
def test_forward_bf16_fast(w, hw, B, zsave):
    """bf16 fast paths (w = 14 on square NCHW 28x28 and 56x56 images, w = 7 on 56x56; table,
    bf16 output; 14x14 goes the general way): batches that fill whole units and ragged ones;
    z_save equals y bit for bit (no mix)."""
    C = 3
    L1 = 2 * w - 1
    say(f"forward bf16 fast w={w} {hw}x{hw} B={B} C={C} zsave={zsave}")
    x = synth.round_to_bf16(synth.normal_f32((B, C, hw, hw), 1.0, seed=31))
    T = synth.round_to_bf16(synth.normal_f32((C, L1, L1), 0.02, seed=32))
    z = torch.empty((B, C, hw, hw), dtype=torch.bfloat16, device="cuda") if zsave else None
    y = R().wbmm_forward(dev_bf16(x), w, T=dev_bf16(T), out_dtype=torch.bfloat16, z_save=z)
    want = O.wbmm_forward(x.astype(np.float64), w, T=T.astype(np.float64))
    assert_bf16(host(y), want, "y")
    if zsave:
        assert torch.equal(z.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("w,hw", [(14, 14), (14, 28), (14, 56), (7, 56), (28, 56)])
def test_forward_bf16_fast_identity_bitwise(w, hw):
    """One-hot table at the centre: M = I, every product is 1 * x or 0 * x and the bf16 output
    reproduces the bf16 input bit for bit (pins the fast path's operand placement)."""
    B, C = 4, 2
    say(f"forward bf16 fast identity w={w} {hw}x{hw}")
    x = synth.round_to_bf16(synth.normal_f32((B, C, hw, hw), 1.0, seed=33))
    T = np.zeros((C, 2 * w - 1, 2 * w - 1), np.float32)
    T[:, w - 1, w - 1] = 1.0
    y = R().wbmm_forward(dev_bf16(x), w, T=dev_bf16(T), out_dtype=torch.bfloat16)
    assert np.array_equal(host(y), x)


def _window_shift(x, w, dy, dx):
    """out[i] = x[(y_i - dy, x_i - dx)] inside each window, zero where that pixel lies outside
    it: the WBMM output for a one-hot table at offset (dy, dx) from the centre, per channel."""
    B, C, H, W = x.shape
    out = np.zeros_like(x)
    for c in range(C):
        for yi in range(w):
            for xi in range(w):
                ys, xs = yi - dy[c], xi - dx[c]
                if 0 <= ys < w and 0 <= xs < w:
                    out[:, c, yi::w, xi::w] = x[:, c, ys::w, xs::w]
    return out


@pytest.mark.parametrize("w,hw,B,C", [(14, 56, 4, 800), (14, 56, 7, 300), (14, 28, 16, 1100),
                                      (7, 56, 4, 900), (7, 56, 5, 300), (28, 56, 17, 40)])
def test_forward_bf16_fast_shift_bitwise(w, hw, B, C):
    _bf16_shift_case(w, hw, B, C, mix=False)


@pytest.mark.parametrize("hw,B,C", [(28, 16, 700), (28, 37, 300), (56, 5, 400)])
def test_forward_bf16_fused_mix_shift_bitwise(hw, B, C):
    """The w = 14 bf16 forward with the 3x3 mix fused: one-hot tables per channel and the identity
    mix make y and z_save the window-shifted input bit for bit, which pins the staging of the
    output tiles, the halo and the column-pair sweep over many units and ragged batches."""
    _bf16_shift_case(14, hw, B, C, mix=True)


@pytest.mark.parametrize("B,C", [(1, 1), (3, 2), (9, 3), (17, 2)])
@pytest.mark.parametrize("mix,zsave", [(False, False), (False, True), (True, False), (True, True)])
def test_forward_f32_w28_fast(B, C, mix, zsave):
    """The fast fp32 w = 28 kernel (56x56 maps, 32-window blocks of 8 images): ragged batches
    (blocks part past the batch), several channels, z_save and the 3x3 mix (a separate pass on
    the kernel's z) against the oracle."""
    say(f"forward f32 w=28 fast B={B} C={C} mix={mix} zsave={zsave}")
    yh, want_y, zh, want_z = fwd_case(B, C, 56, 56, 28, mix=mix, zsave=zsave)
    assert_f32(yh, want_y, "y")
    if zsave:
        assert_f32(zh, want_z, "z")


@pytest.mark.parametrize("B,C", [(1, 1), (3, 2), (5, 7)])
@pytest.mark.parametrize("mix,zsave", [(False, False), (False, True), (True, False), (True, True)])
def test_forward_f32_w7_fast(B, C, mix, zsave):
    """The fast fp32 w = 7 kernel (56x56 maps; persistent waves over (channel, image) planes,
    the table operand in registers per channel): batches and channel counts that leave waves with
    one, several or no planes, z_save and the mix (a separate pass) against the oracle."""
    say(f"forward f32 w=7 fast B={B} C={C} mix={mix} zsave={zsave}")
    yh, want_y, zh, want_z = fwd_case(B, C, 56, 56, 7, mix=mix, zsave=zsave)
    assert_f32(yh, want_y, "y")
    if zsave:
        assert_f32(zh, want_z, "z")


@pytest.mark.parametrize("B,C", [(4, 900), (9, 300), (1, 2050)])
def test_forward_f32_w7_shift_bitwise_all_channels(B, C):
    """One-hot tables at a different offset in every channel: the fast fp32 w = 7 kernel's output
    is the input shifted inside each window, bit for bit. More planes than waves, so waves walk
    several planes and re-form the table operand when the channel changes."""
    w, hw = 7, 56
    say(f"forward f32 w=7 shift all channels B={B} C={C}")
    x = synth.normal_f32((B, C, hw, hw), 1.0, seed=38)
    L1 = 2 * w - 1
    dy = (np.arange(C) * 5 + 1) % L1 - (w - 1)
    dx = (np.arange(C) * 3 + 4) % L1 - (w - 1)
    T = np.zeros((C, L1, L1), np.float32)
    T[np.arange(C), dy + w - 1, dx + w - 1] = 1.0
    want = _window_shift(x, w, dy, dx)
    assert np.array_equal(host(R().wbmm_forward(dev(x), w, T=dev(T))), want)


@pytest.mark.parametrize("B,C", [(10, 300), (8, 129), (3, 520)])
def test_forward_f32_w28_shift_bitwise_all_channels(B, C):
    """One-hot tables at a different offset in every channel: the fast fp32 w = 28 kernel's
    output is the input shifted inside each window, bit for bit, in every channel. More blocks
    than resident workgroups, so workgroups walk several blocks and restage the table when the
    channel changes."""
    w, hw = 28, 56
    say(f"forward f32 w=28 shift all channels B={B} C={C}")
    x = synth.normal_f32((B, C, hw, hw), 1.0, seed=37)
    L1 = 2 * w - 1
    dy = (np.arange(C) * 7 + 2) % L1 - (w - 1)
    dx = (np.arange(C) * 13 + 5) % L1 - (w - 1)
    T = np.zeros((C, L1, L1), np.float32)
    T[np.arange(C), dy + w - 1, dx + w - 1] = 1.0
    want = _window_shift(x, w, dy, dx)
    assert np.array_equal(host(R().wbmm_forward(dev(x), w, T=dev(T))), want)


def _window_shift_padded(x, w, dy, dx):
    """_window_shift on a map zero-padded up to whole windows, cropped back."""
    B, C, H, W = x.shape
    Hp, Wp = -(-H // w) * w, -(-W // w) * w
    xp = np.zeros((B, C, Hp, Wp), x.dtype)
    xp[:, :, :H, :W] = x
    return _window_shift(xp, w, dy, dx)[:, :, :H, :W]


@pytest.mark.parametrize("B,C,H,W", [(2, 3, 128, 128), (1, 2, 30, 25), (3, 2, 14, 20),
                                     (1, 1, 140, 140), (5, 2, 42, 14), (1, 3, 17, 150)])
@pytest.mark.parametrize("mix,zsave", [(False, False), (False, True), (True, False), (True, True)])
def test_forward_f32_tab_fast(B, C, H, W, mix, zsave):
    """The fp32 w = 14 table kernel for maps that are not whole 14/28/56 images (padded, ragged,
    one window wide): z_save and the mix (a separate pass) against the oracle."""
    say(f"forward f32 table fast B={B} C={C} H={H} W={W} mix={mix} zsave={zsave}")
    yh, want_y, zh, want_z = fwd_case(B, C, H, W, 14, mix=mix, zsave=zsave)
    assert_f32(yh, want_y, "y")
    if zsave:
        assert_f32(zh, want_z, "z")


@pytest.mark.parametrize("B,C,H,W", [(2, 300, 128, 128), (3, 129, 30, 44), (1, 520, 60, 70)])
def test_forward_f32_tab_shift_bitwise_all_channels(B, C, H, W):
    """One-hot tables at a different offset in every channel on padded maps: the fp32 w = 14
    table kernel's output is the input shifted inside each window, bit for bit, in every channel.
    More work items than waves, so waves walk several wave-units and thirds and restage their
    table when the channel changes."""
    w = 14
    say(f"forward f32 table shift all channels B={B} C={C} H={H} W={W}")
    x = synth.normal_f32((B, C, H, W), 1.0, seed=39)
    L1 = 2 * w - 1
    dy = (np.arange(C) * 5 + 2) % L1 - (w - 1)
    dx = (np.arange(C) * 11 + 1) % L1 - (w - 1)
    T = np.zeros((C, L1, L1), np.float32)
    T[np.arange(C), dy + w - 1, dx + w - 1] = 1.0
    want = _window_shift_padded(x, w, dy, dx)
    assert np.array_equal(host(R().wbmm_forward(dev(x), w, T=dev(T))), want)


@pytest.mark.parametrize("B,C,H,W", [(2, 300, 128, 128), (1, 130, 45, 33)])
def test_forward_hier_tab_shift_bitwise_all_channels(B, C, H, W):
    """Zero window tables and one-hot 7 x 7 sub-tables at a different offset in every channel:
    the fold on chip of the fp32 table kernel makes the output the input shifted inside each
    7 x 7 sub-window, bit for bit, on padded maps."""
    w, s = 14, 7
    say(f"forward hier table shift all channels B={B} C={C} H={H} W={W}")
    x = synth.normal_f32((B, C, H, W), 1.0, seed=40)
    S1 = 2 * s - 1
    dy = (np.arange(C) * 3 + 1) % S1 - (s - 1)
    dx = (np.arange(C) * 7 + 4) % S1 - (s - 1)
    T = np.zeros((C, 2 * w - 1, 2 * w - 1), np.float32)
    Ts = np.zeros((C, S1, S1), np.float32)
    Ts[np.arange(C), dy + s - 1, dx + s - 1] = 1.0
    want = _window_shift_padded(x, s, dy, dx)
    y = R().wbmm_forward_hier(dev(x), w, s, dev(T), dev(Ts))
    assert np.array_equal(host(y), want)


def _bf16_shift_case(w, hw, B, C, mix):
    """One-hot tables at a different offset in every channel: the output is the input shifted
    inside each window (exact in bf16). More units than resident workgroups, so workgroups walk
    several units and rebuild the staged table when the channel changes."""
    say(f"forward bf16 fast shift w={w} {hw}x{hw} B={B} C={C} mix={mix}")
    x = synth.round_to_bf16(synth.normal_f32((B, C, hw, hw), 1.0, seed=34))
    L1 = 2 * w - 1
    dy = (np.arange(C) * 5) % L1 - (w - 1)
    dx = (np.arange(C) * 11 + 3) % L1 - (w - 1)
    T = np.zeros((C, L1, L1), np.float32)
    T[np.arange(C), dy + w - 1, dx + w - 1] = 1.0
    want = _window_shift(x, w, dy, dx)
    if not mix:
        y = R().wbmm_forward(dev_bf16(x), w, T=dev_bf16(T), out_dtype=torch.bfloat16)
        assert np.array_equal(host(y), want)
        return
    W9 = np.zeros((C, 3, 3), np.float32)
    W9[:, 1, 1] = 1.0
    z = torch.empty((B, C, hw, hw), dtype=torch.bfloat16, device="cuda")
    y = R().wbmm_forward(dev_bf16(x), w, T=dev_bf16(T), mix_w=dev(W9), z_save=z,
                         out_dtype=torch.bfloat16)
    assert np.array_equal(host(z), want)
    assert np.array_equal(host(y), want)


# ----------------------------------------------------------------------------- workloads
def _sample_channels(C, k, seed=0):
    rng = np.random.default_rng(seed + 1000)
    return np.sort(rng.choice(C, size=min(k, C), replace=False))


@pytest.mark.parametrize("cached", [False, True])
def test_workload_stage1_w14_sampled(cached):
    wl = synth.WORKLOADS["stage1_w14"]
    say(f"stage1_w14 full size B={wl.B} C={wl.C} cached={cached}")
    inp = synth.draw_inputs(wl)
    x, T = inp["x"], inp["T"]
    Td = dev(T)
    kw = {"M": R().wbmm_build_matrix(Td, wl.w)} if cached else {"T": Td}
    y = host(R().wbmm_forward(dev(x), wl.w, **kw))
    ch = _sample_channels(wl.C, 6)
    want = O.wbmm_forward(x[:, ch].astype(np.float64), wl.w, T=T[ch].astype(np.float64))
    assert_f32(y[:, ch], want, f"y channels {list(ch)}")


@pytest.mark.parametrize("name", ["bf16_w7", "bf16_w14", "bf16_w28"])
def test_workload_bf16_sweep_sampled(name):
    wl = synth.WORKLOADS[name]
    say(f"{name} full size B={wl.B} C={wl.C}")
    inp = synth.draw_inputs(wl)
    x, T = inp["x"], inp["T"]
    y = host(R().wbmm_forward(dev_bf16(x), wl.w, T=dev_bf16(T)))
    ch = _sample_channels(wl.C, 4)
    want = O.wbmm_forward(x[:, ch].astype(np.float64), wl.w, T=T[ch].astype(np.float64))
    assert_bf16(y[:, ch], want, f"y channels {list(ch)}")


def test_workload_highres_fold_mix():
    wl = synth.WORKLOADS["highres_w14"]
    say(f"highres_w14 B={wl.B} C={wl.C} H={wl.H} fold s={wl.s} + mix")
    inp = synth.draw_inputs(wl)
    x, T, Ts, Wm = inp["x"], inp["T"], inp["T_sub"], inp["Wmix"]
    M = R().wbmm_fold_hier(R().wbmm_build_matrix(dev(T), wl.w), dev(Ts), wl.w, wl.s)
    Mh = host(M)
    Mo = O.fold_hier(O.build_matrix(T, wl.w), Ts, wl.w, wl.s)
    assert np.array_equal(Mh, Mo)
    zs = torch.empty(x.shape, dtype=torch.float32, device="cuda")
    y = R().wbmm_forward(dev(x), wl.w, M=M, mix_w=dev(Wm), z_save=zs)
    want_y, want_z = O.layer_forward(x.astype(np.float64), wl.w, M=Mo, Wmix=Wm)
    assert_f32(host(zs), want_z, "z")
    assert_f32(host(y), want_y, "y")


# ----------------------------------------------------------------------------- backward
def bwd_case(B, C, H, W, w, *, mix, cached=False, layout="NCHW", seed=0):
    x = synth.normal_f32((B, C, H, W), 1.0, seed=seed)
    T = synth.normal_f32((C, 2 * w - 1, 2 * w - 1), 0.02, seed=seed + 1)
    Wm = synth.normal_f32((C, 3, 3), 0.1, seed=seed + 2) if mix else None
    dy = synth.normal_f32((B, C, H, W), 1.0, seed=seed + 3)
    to_l = (lambda a: a) if layout == "NCHW" else (lambda a: a.transpose(0, 2, 3, 1))
    from_l = (lambda a: a) if layout == "NCHW" else (lambda a: a.transpose(0, 3, 1, 2))
    xd, dyd, Td = dev(to_l(x)), dev(to_l(dy)), dev(T)
    kw = {"M": R().wbmm_build_matrix(Td, w)} if cached else {"T": Td}
    Wd = dev(Wm) if mix else None
    zs = torch.empty_like(xd) if mix else None
    R().wbmm_forward(xd, w, mix_w=Wd, z_save=zs, layout=layout, **kw)
    dx, dT, dW = R().wbmm_backward(xd, dyd, w, mix_w=Wd, z_saved=zs, layout=layout, **kw)
    # the oracle's backward uses the z the GPU saved (fp32), as the GPU does
    z_used = from_l(host(zs)).astype(np.float64) if mix else None
    wdx, wdT, wdW = O.layer_backward(x.astype(np.float64), dy.astype(np.float64), w,
                                     T=T.astype(np.float64), Wmix=Wm, z=z_used)
    return (from_l(host(dx)), host(dT), host(dW) if mix else None), (wdx, wdT, wdW)


@pytest.mark.parametrize("B,C,H,W,w,mix", [
    (2, 3, 28, 28, 14, True), (2, 3, 28, 28, 14, False), (3, 2, 10, 13, 4, True),
    (1, 2, 7, 7, 7, False), (2, 2, 21, 14, 7, True), (2, 1, 4, 4, 1, True),
    (1, 2, 30, 30, 15, False), (1, 2, 32, 32, 16, True), (1, 2, 100, 100, 14, True),
    (1, 2, 128, 128, 14, True), (2, 2, 128, 120, 14, False),
    (2, 2, 17, 23, 5, False),
    # the fast fp32 kernels on 56x56 and 14x14 images (ragged batches: last unit part empty)
    (2, 3, 56, 56, 14, True), (2, 3, 56, 56, 14, False), (5, 3, 56, 56, 14, True),
    (5, 3, 14, 14, 14, True), (5, 3, 14, 14, 14, False), (70, 2, 14, 14, 14, True),
    # the direct mix adjoint pass on ragged plane heights (last row run part empty), several
    # chunks per plane
    (1, 2, 150, 74, 14, True), (3, 2, 26, 30, 5, True),
])
@pytest.mark.parametrize("cached", [False, True])
def test_backward_shapes(B, C, H, W, w, mix, cached):
    say(f"backward B={B} C={C} H={H} W={W} w={w} mix={mix} cached={cached}")
    (dx, dT, dW), (wdx, wdT, wdW) = bwd_case(B, C, H, W, w, mix=mix, cached=cached)
    assert_f32(dx, wdx, "dx")
    assert_f32(dT, wdT, "dT")
    if mix:
        assert_f32(dW, wdW, "dWmix")


@pytest.mark.parametrize("B,C,H,W,w,mix,layout", [
    (2, 2, 28, 28, 28, True, "NCHW"), (2, 2, 28, 28, 28, False, "NCHW"),
    (3, 2, 56, 56, 28, True, "NCHW"),    # dx on the fast fp32 w = 28 kernel
    (1, 3, 40, 37, 20, True, "NCHW"),    # ragged, padded map
    (2, 2, 64, 64, 32, False, "NCHW"), (3, 2, 30, 45, 17, True, "NCHW"),
    (2, 2, 28, 28, 28, True, "NHWC"), (1, 2, 33, 21, 19, False, "NHWC"),
])
@pytest.mark.parametrize("cached", [False, True])
def test_backward_wide(B, C, H, W, w, mix, layout, cached):
    """The backward for windows wider than 16 (dx through the forward with M^T: the rotated table,
    or the transposed cached matrix; dT on 32x32 row-pair tiles) against the oracle, with the mix
    and without, padded and ragged maps, NHWC; run twice, bitwise equal."""
    say(f"backward wide B={B} C={C} H={H} W={W} w={w} mix={mix} {layout} cached={cached}")
    (dx, dT, dW), (wdx, wdT, wdW) = bwd_case(B, C, H, W, w, mix=mix, cached=cached, layout=layout)
    assert_f32(dx, wdx, "dx")
    assert_f32(dT, wdT, "dT")
    if mix:
        assert_f32(dW, wdW, "dWmix")
    (dx2, dT2, _), _ = bwd_case(B, C, H, W, w, mix=mix, cached=cached, layout=layout)
    assert np.array_equal(dx, dx2) and np.array_equal(dT, dT2)


def test_backward_nhwc():
    say("backward NHWC B=2 C=3 28x28 w=14 mix")
    (dx, dT, dW), (wdx, wdT, wdW) = bwd_case(2, 3, 28, 28, 14, mix=True, layout="NHWC")
    assert_f32(dx, wdx, "dx")
    assert_f32(dT, wdT, "dT")
    assert_f32(dW, wdW, "dWmix")


def test_workload_train_w14_full():
    """The training workload at full size: every output against the oracle, plus determinism."""
    wl = synth.WORKLOADS["train_w14"]
    say(f"train_w14 full B={wl.B} C={wl.C} H={wl.H} w={wl.w} fwd+bwd")
    inp = synth.draw_inputs(wl)
    x, T, Wm, dy = inp["x"], inp["T"], inp["Wmix"], inp["dY"]
    xd, Td, Wd, dyd = dev(x), dev(T), dev(Wm), dev(dy)
    zs = torch.empty_like(xd)
    y = R().wbmm_forward(xd, wl.w, T=Td, mix_w=Wd, z_save=zs)
    ws = torch.zeros(R().wbmm_backward_workspace_bytes(wl.B, wl.C, wl.H, wl.W, wl.w, has_mix=True),
                     dtype=torch.uint8, device="cuda")
    dx, dT, dW = R().wbmm_backward(xd, dyd, wl.w, T=Td, mix_w=Wd, z_saved=zs, workspace=ws)
    want_y, want_z = O.layer_forward(x.astype(np.float64), wl.w, T=T.astype(np.float64), Wmix=Wm)
    assert_f32(host(y), want_y, "y")
    assert_f32(host(zs), want_z, "z")
    wdx, wdT, wdW = O.layer_backward(x.astype(np.float64), dy.astype(np.float64), wl.w,
                                     T=T.astype(np.float64), Wmix=Wm, z=host(zs).astype(np.float64))
    assert_f32(host(dx), wdx, "dx")
    assert_f32(host(dT), wdT, "dT")
    assert_f32(host(dW), wdW, "dWmix")
    # run twice: bitwise identical (fixed-order reductions; workspace reused)
    y2 = R().wbmm_forward(xd, wl.w, T=Td, mix_w=Wd)
    dx2, dT2, dW2 = R().wbmm_backward(xd, dyd, wl.w, T=Td, mix_w=Wd, z_saved=zs, workspace=ws)
    assert torch.equal(y, y2) and torch.equal(dx, dx2)
    assert torch.equal(dT, dT2) and torch.equal(dW, dW2)


def test_backward_partial_outputs():
    say("backward partial outputs (dT only, dx only)")
    B, C, H, W, w = 2, 3, 28, 28, 14
    x = synth.normal_f32((B, C, H, W), 1.0, seed=11)
    T = synth.normal_f32((C, 27, 27), 0.02, seed=12)
    dy = synth.normal_f32((B, C, H, W), 1.0, seed=13)
    _, dT, _ = R().wbmm_backward(dev(x), dev(dy), w, T=dev(T), dx=False)
    dx, dT2, _ = R().wbmm_backward(dev(x), dev(dy), w, T=dev(T), dT=False)
    assert dT2 is None
    wdx, wdT, _ = O.layer_backward(x.astype(np.float64), dy.astype(np.float64), w, T=T.astype(np.float64))
    assert_f32(host(dT), wdT, "dT")
    assert_f32(host(dx), wdx, "dx")


def test_errors_enqueue_nothing():
    """Invalid calls fail on the host with a message and leave outputs untouched."""
    say("error paths")
    Rm = R()
    x = torch.zeros((1, 2, 8, 8), device="cuda")
    y = torch.full_like(x, 7.0)
    T = torch.zeros((2, 7, 7), device="cuda")
    with pytest.raises(Rm.WbmmError) as e:
        Rm.wbmm_forward(x, 4, T=T, M=Rm.wbmm_build_matrix(T, 4), y=y)
    assert e.value.status == Rm.WBMM_E_INVALID
    with pytest.raises(Rm.WbmmError) as e:
        Rm.wbmm_forward(x, 33, T=T, y=y)
    assert e.value.status == Rm.WBMM_E_INVALID
    with pytest.raises(Rm.WbmmError) as e:
        Rm.wbmm_forward(x, 4, T=T, y=x)  # y aliases x
    assert e.value.status == Rm.WBMM_E_INVALID
    with pytest.raises(Rm.WbmmError) as e:
        Rm.wbmm_backward(x, x, 33, T=torch.zeros((2, 65, 65), device="cuda"))
    assert e.value.status == Rm.WBMM_E_INVALID
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)


# ----------------------------------------------------------------------------- hierarchical fold
def hier_inputs(B, C, H, W, w, s, seed, mix):
    x = synth.normal_f32((B, C, H, W), 1.0, seed=seed)
    T = synth.normal_f32((C, 2 * w - 1, 2 * w - 1), 0.02, seed=seed + 1)
    Ts = synth.normal_f32((C, 2 * s - 1, 2 * s - 1), 0.02, seed=seed + 2)
    Wm = synth.normal_f32((C, 3, 3), 0.1, seed=seed + 3) if mix else None
    return x, T, Ts, Wm


@pytest.mark.parametrize("B,C,H,W,w,s", [(2, 3, 28, 28, 14, 7), (1, 2, 30, 25, 14, 7),
                                         (2, 3, 8, 8, 4, 2), (1, 2, 12, 18, 6, 3),
                                         (2, 2, 16, 16, 8, 4), (1, 2, 128, 128, 14, 7)])
@pytest.mark.parametrize("mix", [False, True])
def test_forward_hier(B, C, H, W, w, s, mix):
    """The fold on chip (image and window mode, ragged maps) against the oracle's explicit fold."""
    say(f"forward hier B={B} C={C} H={H} W={W} w={w} s={s} mix={mix}")
    x, T, Ts, Wm = hier_inputs(B, C, H, W, w, s, 70, mix)
    zs = torch.empty((B, C, H, W), device="cuda")
    y = R().wbmm_forward_hier(dev(x), w, s, dev(T), dev(Ts), mix_w=dev(Wm) if mix else None,
                              z_save=zs)
    want_y, want_z = O.layer_forward_hier(x.astype(np.float64), w, s, T, Ts, Wmix=Wm)
    assert_f32(host(y), want_y, "y")
    assert_f32(host(zs), want_z, "z")


@pytest.mark.parametrize("w,s", [(14, 7), (4, 2)])
def test_forward_hier_one_hot_bitwise(w, s):
    """One-hot T and T_sub at different offsets per channel: every output is a sum of at most two
    input pixels with weight 1 (or one with weight 2), exact in fp32, so the on-chip fold must
    match the oracle's explicit fold bit for bit."""
    B, C, H, W = 3, 5, 2 * w, 3 * w
    say(f"forward hier one-hot w={w} s={s}")
    x = synth.normal_f32((B, C, H, W), 1.0, seed=75)
    L1, Ls = 2 * w - 1, 2 * s - 1
    T = np.zeros((C, L1, L1), np.float32)
    Ts = np.zeros((C, Ls, Ls), np.float32)
    c = np.arange(1, C)
    T[c, (c * 3) % L1, (c * 7 + 1) % L1] = 1.0
    Ts[c, (c * 2 + 1) % Ls, (c * 5) % Ls] = 1.0
    T[0, w - 1, w - 1] = 1.0  # channel 0: both at offset 0 -> z = 2 x
    Ts[0, s - 1, s - 1] = 1.0
    y = R().wbmm_forward_hier(dev(x), w, s, dev(T), dev(Ts))
    want, _ = O.layer_forward_hier(x.astype(np.float64), w, s, T, Ts)
    assert np.array_equal(host(y), want.astype(np.float32))


@pytest.mark.parametrize("B,C,H,W,w,s", [(2, 3, 28, 28, 14, 7), (1, 2, 30, 25, 14, 7),
                                         (2, 3, 8, 8, 4, 2), (1, 2, 12, 18, 6, 3),
                                         (2, 2, 16, 16, 8, 4), (1, 2, 128, 128, 14, 7)])
@pytest.mark.parametrize("mix", [False, True])
def test_backward_hier(B, C, H, W, w, s, mix):
    """dx, dT, dT_sub (and dWmix) of the folded layer against the oracle; image mode fuses the mix
    adjoint, window mode (128x128) runs it as separate passes. Determinism: a second call is
    bitwise identical."""
    say(f"backward hier B={B} C={C} H={H} W={W} w={w} s={s} mix={mix}")
    x, T, Ts, Wm = hier_inputs(B, C, H, W, w, s, 80, mix)
    dy = synth.normal_f32((B, C, H, W), 1.0, seed=85)
    xd, Td, Tsd, dyd = dev(x), dev(T), dev(Ts), dev(dy)
    Wd = dev(Wm) if mix else None
    zs = None
    if mix:
        zs = torch.empty_like(xd)
        R().wbmm_forward_hier(xd, w, s, Td, Tsd, mix_w=Wd, z_save=zs)
    dx, dT, dTs, dW = R().wbmm_backward_hier(xd, dyd, w, s, Td, Tsd, mix_w=Wd, z_saved=zs)
    z64 = host(zs).astype(np.float64) if mix else None
    wdx, wdT, wdTs, wdW = O.layer_backward_hier(x.astype(np.float64), dy.astype(np.float64), w, s,
                                                T, Ts, Wmix=Wm, z=z64)
    assert_f32(host(dx), wdx, "dx")
    assert_f32(host(dT), wdT, "dT")
    assert_f32(host(dTs), wdTs, "dT_sub")
    if mix:
        assert_f32(host(dW), wdW, "dWmix")
    dx2, dT2, dTs2, _ = R().wbmm_backward_hier(xd, dyd, w, s, Td, Tsd, mix_w=Wd, z_saved=zs)
    assert torch.equal(dx, dx2) and torch.equal(dT, dT2) and torch.equal(dTs, dTs2)


def test_backward_hier_partial_outputs():
    """Only dT_sub, or only dx: the skipped outputs stay untouched and the others match."""
    B, C, H, W, w, s = 2, 3, 28, 28, 14, 7
    say("backward hier partial outputs")
    x, T, Ts, _ = hier_inputs(B, C, H, W, w, s, 90, False)
    dy = synth.normal_f32((B, C, H, W), 1.0, seed=95)
    xd, Td, Tsd, dyd = dev(x), dev(T), dev(Ts), dev(dy)
    _, dT0, dTs, _ = R().wbmm_backward_hier(xd, dyd, w, s, Td, Tsd, dx=False, dT=False)
    assert dT0 is None
    dx, _, dTs0, _ = R().wbmm_backward_hier(xd, dyd, w, s, Td, Tsd, dT=False, dT_sub=False)
    assert dTs0 is None
    wdx, _, wdTs, _ = O.layer_backward_hier(x.astype(np.float64), dy.astype(np.float64), w, s, T, Ts)
    assert_f32(host(dTs), wdTs, "dT_sub")
    assert_f32(host(dx), wdx, "dx")


# Sub-windows other than the quadrants (s | w, w != 2s) and w = 2s above 16: M' is folded in the
# workspace and the cached-matrix kernels run on it; dT_sub is the table gradient of an s-window
# layer on the same map gradient.
HIER_GENERAL = [(2, 3, 24, 24, 12, 4, "NCHW"), (1, 2, 26, 20, 12, 3, "NCHW"),
                (2, 2, 28, 28, 14, 2, "NCHW"), (1, 2, 33, 30, 16, 4, "NHWC"),
                (1, 2, 36, 36, 18, 9, "NCHW"), (1, 2, 40, 40, 20, 10, "NCHW"),
                (1, 2, 15, 20, 10, 1, "NCHW")]


def _to_layout(a, layout):
    return a if layout == "NCHW" else np.ascontiguousarray(a.transpose(0, 2, 3, 1))


def _from_layout(a, layout):
    return a if layout == "NCHW" else a.transpose(0, 3, 1, 2)


@pytest.mark.parametrize("B,C,H,W,w,s,layout", HIER_GENERAL)
@pytest.mark.parametrize("mix", [False, True])
def test_forward_hier_general(B, C, H, W, w, s, layout, mix):
    """The fold for any s dividing w against the oracle's explicit fold (ragged and padded maps,
    one channels-last case)."""
    say(f"forward hier general B={B} C={C} H={H} W={W} w={w} s={s} {layout} mix={mix}")
    x, T, Ts, Wm = hier_inputs(B, C, H, W, w, s, 170, mix)
    xd = dev(_to_layout(x, layout))
    zs = torch.empty_like(xd)
    y = R().wbmm_forward_hier(xd, w, s, dev(T), dev(Ts), mix_w=dev(Wm) if mix else None,
                              layout=layout, z_save=zs)
    want_y, want_z = O.layer_forward_hier(x.astype(np.float64), w, s, T, Ts, Wmix=Wm)
    assert_f32(_from_layout(host(y), layout), want_y, "y")
    assert_f32(_from_layout(host(zs), layout), want_z, "z")


@pytest.mark.parametrize("w,s", [(12, 3), (20, 10)])
def test_forward_hier_general_one_hot_bitwise(w, s):
    """One-hot T and T_sub (at offset 0 on channel 0, so that matrix entries of 2 appear): the
    folded matrix holds 0, 1 and 2, every output is exact in fp32 and must match bit for bit."""
    B, C, H, W = 2, 4, 2 * w, 2 * w + s
    say(f"forward hier general one-hot w={w} s={s}")
    x = synth.normal_f32((B, C, H, W), 1.0, seed=175)
    L1, Ls = 2 * w - 1, 2 * s - 1
    T = np.zeros((C, L1, L1), np.float32)
    Ts = np.zeros((C, Ls, Ls), np.float32)
    c = np.arange(1, C)
    T[c, (c * 5) % L1, (c * 3 + 2) % L1] = 1.0
    Ts[c, (c * 2) % Ls, (c + 1) % Ls] = 1.0
    T[0, w - 1, w - 1] = 1.0
    Ts[0, s - 1, s - 1] = 1.0
    y = R().wbmm_forward_hier(dev(x), w, s, dev(T), dev(Ts))
    want, _ = O.layer_forward_hier(x.astype(np.float64), w, s, T, Ts)
    assert np.array_equal(host(y), want.astype(np.float32))


@pytest.mark.parametrize("B,C,H,W,w,s,layout", HIER_GENERAL)
@pytest.mark.parametrize("mix", [False, True])
def test_backward_hier_general(B, C, H, W, w, s, layout, mix):
    """dx, dT, dT_sub (and dWmix) for any s dividing w against the oracle; a second call is
    bitwise identical."""
    say(f"backward hier general B={B} C={C} H={H} W={W} w={w} s={s} {layout} mix={mix}")
    x, T, Ts, Wm = hier_inputs(B, C, H, W, w, s, 180, mix)
    dy = synth.normal_f32((B, C, H, W), 1.0, seed=185)
    xd, dyd = dev(_to_layout(x, layout)), dev(_to_layout(dy, layout))
    Td, Tsd = dev(T), dev(Ts)
    Wd = dev(Wm) if mix else None
    zs = None
    if mix:
        zs = torch.empty_like(xd)
        R().wbmm_forward_hier(xd, w, s, Td, Tsd, mix_w=Wd, layout=layout, z_save=zs)
    dx, dT, dTs, dW = R().wbmm_backward_hier(xd, dyd, w, s, Td, Tsd, mix_w=Wd, z_saved=zs,
                                             layout=layout)
    z64 = _from_layout(host(zs), layout).astype(np.float64) if mix else None
    wdx, wdT, wdTs, wdW = O.layer_backward_hier(x.astype(np.float64), dy.astype(np.float64), w, s,
                                                T, Ts, Wmix=Wm, z=z64)
    assert_f32(_from_layout(host(dx), layout), wdx, "dx")
    assert_f32(host(dT), wdT, "dT")
    assert_f32(host(dTs), wdTs, "dT_sub")
    if mix:
        assert_f32(host(dW), wdW, "dWmix")
    dx2, dT2, dTs2, _ = R().wbmm_backward_hier(xd, dyd, w, s, Td, Tsd, mix_w=Wd, z_saved=zs,
                                               layout=layout)
    assert torch.equal(dx, dx2) and torch.equal(dT, dT2) and torch.equal(dTs, dTs2)


def test_backward_hier_general_partial_outputs():
    """General s: only dT_sub (the main backward is skipped), or only dx (no sub backward)."""
    B, C, H, W, w, s = 2, 2, 24, 24, 12, 4
    say("backward hier general partial outputs")
    x, T, Ts, _ = hier_inputs(B, C, H, W, w, s, 190, False)
    dy = synth.normal_f32((B, C, H, W), 1.0, seed=195)
    xd, Td, Tsd, dyd = dev(x), dev(T), dev(Ts), dev(dy)
    _, dT0, dTs, _ = R().wbmm_backward_hier(xd, dyd, w, s, Td, Tsd, dx=False, dT=False)
    assert dT0 is None
    dx, _, dTs0, _ = R().wbmm_backward_hier(xd, dyd, w, s, Td, Tsd, dT=False, dT_sub=False)
    assert dTs0 is None
    wdx, _, wdTs, _ = O.layer_backward_hier(x.astype(np.float64), dy.astype(np.float64), w, s, T, Ts)
    assert_f32(host(dTs), wdTs, "dT_sub")
    assert_f32(host(dx), wdx, "dx")


@pytest.mark.parametrize("B,C,H", [(5, 3, 14), (18, 2, 28), (5, 2, 56)])
@pytest.mark.parametrize("mix", [False, True])
def test_hier_fast_shapes(B, C, H, mix):
    """w = 14, s = 7 on the whole-image shapes (14², 28², 56² NCHW), where the fold runs in the
    fast kernels: the folded copy picked per output quadrant and the sub-window band chains of
    the table gradient. Ragged batches leave the last unit part empty."""
    w, s = 14, 7
    say(f"hier fast shapes B={B} C={C} H=W={H} mix={mix}")
    x, T, Ts, Wm = hier_inputs(B, C, H, H, w, s, 100, mix)
    dy = synth.normal_f32((B, C, H, H), 1.0, seed=105)
    xd, Td, Tsd, dyd = dev(x), dev(T), dev(Ts), dev(dy)
    Wd = dev(Wm) if mix else None
    zs = torch.empty_like(xd)
    y = R().wbmm_forward_hier(xd, w, s, Td, Tsd, mix_w=Wd, z_save=zs)
    want_y, want_z = O.layer_forward_hier(x.astype(np.float64), w, s, T, Ts, Wmix=Wm)
    assert_f32(host(y), want_y, "y")
    assert_f32(host(zs), want_z, "z")
    dx, dT, dTs, dW = R().wbmm_backward_hier(xd, dyd, w, s, Td, Tsd, mix_w=Wd,
                                             z_saved=zs if mix else None)
    z64 = host(zs).astype(np.float64) if mix else None
    wdx, wdT, wdTs, wdW = O.layer_backward_hier(x.astype(np.float64), dy.astype(np.float64), w, s,
                                                T, Ts, Wmix=Wm, z=z64)
    assert_f32(host(dx), wdx, "dx")
    assert_f32(host(dT), wdT, "dT")
    assert_f32(host(dTs), wdTs, "dT_sub")
    if mix:
        assert_f32(host(dW), wdW, "dWmix")


def test_hier_fast_one_hot_bitwise():
    """Fast-kernel fold on 28² images: one-hot T and T_sub per channel make every output a sum of
    at most two inputs with weight 1 (channel 0: one input with weight 2), exact in fp32."""
    w, s, B, C, H = 14, 7, 6, 5, 28
    say("hier fast one-hot")
    x = synth.normal_f32((B, C, H, H), 1.0, seed=110)
    T = np.zeros((C, 27, 27), np.float32)
    Ts = np.zeros((C, 13, 13), np.float32)
    c = np.arange(1, C)
    T[c, (c * 5) % 27, (c * 11 + 2) % 27] = 1.0
    Ts[c, (c * 3 + 2) % 13, (c * 4) % 13] = 1.0
    T[0, 13, 13] = 1.0
    Ts[0, 6, 6] = 1.0
    y = R().wbmm_forward_hier(dev(x), w, s, dev(T), dev(Ts))
    want, _ = O.layer_forward_hier(x.astype(np.float64), w, s, T, Ts)
    assert np.array_equal(host(y), want.astype(np.float32))


def test_hier_fast_zero_sub_table_matches_plain():
    """With T_sub = 0 the folded copy equals T, so the hierarchical fast forward and dX are bitwise
    the plain kernels' results; dT (its sub-window band pairs summed in chains of their own) and
    dT_sub (the plain layer's gradient summed over same-sub-window pairs) match the oracle."""
    w, s, B, C, H = 14, 7, 20, 3, 28
    say("hier fast zero sub-table")
    x, T, _, Wm = hier_inputs(B, C, H, H, w, s, 120, True)
    Ts = np.zeros((C, 13, 13), np.float32)
    dy = synth.normal_f32((B, C, H, H), 1.0, seed=125)
    xd, Td, Tsd, dyd, Wd = dev(x), dev(T), dev(Ts), dev(dy), dev(Wm)
    zh, zp = torch.empty_like(xd), torch.empty_like(xd)
    yh = R().wbmm_forward_hier(xd, w, s, Td, Tsd, mix_w=Wd, z_save=zh)
    yp = R().wbmm_forward(xd, w, T=Td, mix_w=Wd, z_save=zp)
    assert torch.equal(yh, yp) and torch.equal(zh, zp)
    dxh, dTh, dTsh, dWh = R().wbmm_backward_hier(xd, dyd, w, s, Td, Tsd, mix_w=Wd, z_saved=zh)
    dxp, dTp, dWp = R().wbmm_backward(xd, dyd, w, T=Td, mix_w=Wd, z_saved=zp)
    assert torch.equal(dxh, dxp) and torch.equal(dWh, dWp)
    _, wdT, wdTs, _ = O.layer_backward_hier(x.astype(np.float64), dy.astype(np.float64), w, s, T,
                                            Ts, Wmix=Wm, z=host(zh).astype(np.float64))
    assert_f32(host(dTh), wdT, "dT")
    assert_f32(host(dTsh), wdTs, "dT_sub")


# ----------------------------------------------------------------------------- DW-Std comparison
@pytest.mark.parametrize("k", [3, 5, 7, 9, 11, 13])
@pytest.mark.parametrize("B,C,H,W", [(2, 3, 56, 56), (2, 5, 28, 28), (1, 2, 13, 17),
                                     (1, 3, 5, 3), (1, 2, 150, 64), (3, 2, 14, 14)])
def test_dwconv_parity(k, B, C, H, W):
    """The k x k depthwise convolution against the oracle: whole 56² / 28² planes (16-byte
    staging and stores, 7- and 4-row tiles), ragged odd widths, maps smaller than the kernel,
    several row bands per plane, several planes per workgroup."""
    say(f"dwconv k={k} B={B} C={C} H={H} W={W}")
    x = synth.normal_f32((B, C, H, W), 1.0, seed=200 + k)
    Wd = synth.normal_f32((C, k, k), 0.05, seed=201 + k)
    y = R().wbmm_dwconv_forward(dev(x), dev(Wd))
    assert_f32(host(y), O.dw_conv_forward(x.astype(np.float64), Wd), "y")


@pytest.mark.parametrize("k", [5, 13])
def test_dwconv_one_hot_is_exact_shift(k):
    """One tap per channel (a different one in each): y is x shifted, bit for bit."""
    B, C, H, W = 2, 6, 28, 36
    say(f"dwconv one-hot k={k}")
    x = synth.normal_f32((B, C, H, W), 1.0, seed=210)
    Wd = np.zeros((C, k, k), np.float32)
    for c in range(C):
        Wd[c, (c * 3) % k, (c * 5 + 1) % k] = 1.0
    y = R().wbmm_dwconv_forward(dev(x), dev(Wd))
    assert np.array_equal(host(y), O.dw_conv_forward(x.astype(np.float64), Wd).astype(np.float32))


@pytest.mark.parametrize("w", [3, 5, 7])
def test_dwconv_on_one_window_matches_wbmm(w):
    """On maps that are exactly one window, DW-Std with k = 2w-1 and the rotated table is WBMM:
    the two GPU operators agree (to rounding) on the same inputs."""
    B, C = 4, 3
    say(f"dwconv vs wbmm on one window w={w}")
    x = synth.normal_f32((B, C, w, w), 1.0, seed=220 + w)
    T = synth.normal_f32((C, 2 * w - 1, 2 * w - 1), 0.05, seed=221 + w)
    y_dw = R().wbmm_dwconv_forward(dev(x), dev(np.ascontiguousarray(T[:, ::-1, ::-1])))
    y_wb = R().wbmm_forward(dev(x), w, T=dev(T))
    assert_f32(host(y_dw), host(y_wb).astype(np.float64), "dw vs wbmm")


def test_dwconv_full_size_sampled():
    """The comparison shape (B=128, C=256, 56², k=13): sampled planes against the oracle."""
    B, C, H, W, k = 128, 256, 56, 56, 13
    say("dwconv full size k=13")
    xn = synth.normal_f32((B, C, H, W), 1.0, seed=230)
    wn = synth.normal_f32((C, k, k), 0.05, seed=231)
    y = host(R().wbmm_dwconv_forward(dev(xn), dev(wn)))
    for b, c in [(0, 0), (127, 255), (64, 3), (5, 200), (100, 129)]:
        want = O.dw_conv_forward(xn[b:b + 1, c:c + 1].astype(np.float64), wn[c:c + 1])
        assert_f32(y[b:b + 1, c:c + 1], want, f"plane ({b},{c})")


# ----------------------------------------------------------------------------- shifted window grid
# w = 14 with a table runs the repacked fast kernels (a cached matrix, other w: general kernels);
# B = 5 at 28x28 leaves 45 windows: 12 repacked images, the last with 3 zero windows
SHIFT_CASES = [(2, 3, 28, 28, 14, 7, 7), (1, 2, 30, 25, 14, 3, 11), (2, 3, 17, 13, 4, 2, 1),
               (1, 2, 128, 128, 14, 7, 7), (2, 2, 9, 9, 7, 0, 3), (5, 4, 28, 28, 14, 7, 7),
               (3, 2, 5, 40, 14, 13, 0), (1, 2, 40, 40, 20, 10, 10), (2, 3, 42, 36, 14, 6, 4),
               (1, 2, 14, 14, 14, 1, 13), (17, 3, 28, 28, 14, 7, 0), (3, 2, 28, 28, 14, 0, 7),
               (2, 3, 56, 56, 14, 7, 7), (5, 2, 56, 56, 14, 0, 7), (70, 2, 14, 14, 14, 7, 7),
               (3, 2, 14, 14, 14, 7, 0)]


def _window_shift_grid(x, w, oy, ox, dy, dx):
    """_window_shift on the offset grid: the map placed at (oy, ox) in a zero canvas of whole
    windows, shifted inside each window, cropped back."""
    B, C, H, W = x.shape
    Hp, Wp = -(-(H + oy) // w) * w, -(-(W + ox) // w) * w
    xp = np.zeros((B, C, Hp, Wp), x.dtype)
    xp[:, :, oy:oy + H, ox:ox + W] = x
    return _window_shift(xp, w, dy, dx)[:, :, oy:oy + H, ox:ox + W]


@pytest.mark.parametrize("B,C,H,W,oy,ox", [(4, 300, 28, 28, 7, 7), (3, 129, 30, 44, 5, 9),
                                           (2, 130, 40, 36, 6, 4), (1, 260, 17, 13, 13, 0),
                                           (2, 140, 128, 128, 7, 7), (17, 40, 28, 28, 7, 0),
                                           (33, 24, 28, 28, 0, 7), (16, 33, 28, 28, 7, 7),
                                           (3, 40, 56, 56, 7, 7), (17, 24, 56, 56, 7, 0),
                                           (2, 33, 56, 56, 0, 7), (65, 20, 14, 14, 7, 7),
                                           (5, 24, 14, 14, 0, 7)])
def test_forward_shifted_tab_bitwise_all_channels(B, C, H, W, oy, ox):
    """One-hot tables at a different offset in every channel on an offset window grid: the fp32
    w = 14 kernels' output (the table kernel; for offsets of 0 or 7 on 28x28 maps the rolled-map
    kernel, whose masked matrix must drop every pair across pieces) is the input shifted inside
    each window of that grid, bit for bit, in every channel (whole and border windows, even and
    odd column offsets, full and partial units of 16 images)."""
    w = 14
    say(f"forward shifted table shift all channels B={B} C={C} H={H} W={W} o=({oy},{ox})")
    x = synth.normal_f32((B, C, H, W), 1.0, seed=41)
    L1 = 2 * w - 1
    dy = (np.arange(C) * 5 + 3) % L1 - (w - 1)
    dx = (np.arange(C) * 11 + 2) % L1 - (w - 1)
    T = np.zeros((C, L1, L1), np.float32)
    T[np.arange(C), dy + w - 1, dx + w - 1] = 1.0
    want = _window_shift_grid(x, w, oy, ox, dy, dx)
    assert np.array_equal(host(R().wbmm_forward_shifted(dev(x), w, oy, ox, T=dev(T))), want)


@pytest.mark.parametrize("B,C,H,W,w,oy,ox", SHIFT_CASES)
@pytest.mark.parametrize("mix", [False, True])
@pytest.mark.parametrize("src", ["T", "M"])
@pytest.mark.parametrize("zsave", [True, False])
def test_forward_shifted(B, C, H, W, w, oy, ox, mix, src, zsave):
    """Interleaved grid (offset windows, zero border pixels) against the oracle: image and window
    mode, ragged maps, table and cached matrix, with and without the 3x3 mix; without z_save
    the pre-mix map goes through the workspace."""
    say(f"forward shifted B={B} C={C} H={H} W={W} w={w} o=({oy},{ox}) mix={mix} src={src} "
        f"zsave={zsave}")
    x = synth.normal_f32((B, C, H, W), 1.0, seed=240)
    T = synth.normal_f32((C, 2 * w - 1, 2 * w - 1), 0.05, seed=241)
    Wm = synth.normal_f32((C, 3, 3), 0.1, seed=242) if mix else None
    kw = {"T": dev(T)} if src == "T" else {"M": R().wbmm_build_matrix(dev(T), w)}
    zs = torch.empty((B, C, H, W), device="cuda") if zsave else None
    y = R().wbmm_forward_shifted(dev(x), w, oy, ox, mix_w=dev(Wm) if mix else None, z_save=zs,
                                 **kw)
    want_y, want_z = O.layer_forward_shifted(x.astype(np.float64), w, oy, ox, T=T, Wmix=Wm)
    assert_f32(host(y), want_y, "y")
    if zsave:
        assert_f32(host(zs), want_z, "z")


@pytest.mark.parametrize("B,C,H,W,w,oy,ox", [(2, 3, 28, 28, 14, 7, 7), (1, 2, 17, 13, 4, 2, 1),
                                             (1, 2, 56, 56, 14, 5, 9), (5, 4, 28, 28, 14, 7, 7),
                                             (3, 2, 5, 40, 14, 13, 0), (1, 2, 40, 40, 20, 10, 10)])
@pytest.mark.parametrize("zsave", [True, False])
def test_forward_shifted_bf16(B, C, H, W, w, oy, ox, zsave):
    """bf16 maps on the offset grid (w = 14: repacked windows on the fast bf16 forward); z_save,
    without the mix, holds y; without z_save only y is scattered back."""
    say(f"forward shifted bf16 B={B} C={C} H={H} W={W} w={w} o=({oy},{ox}) zsave={zsave}")
    x = synth.round_to_bf16(synth.normal_f32((B, C, H, W), 1.0, seed=245))
    T = synth.round_to_bf16(synth.normal_f32((C, 2 * w - 1, 2 * w - 1), 0.05, seed=246))
    zs = torch.empty((B, C, H, W), device="cuda", dtype=torch.bfloat16) if zsave else None
    y = R().wbmm_forward_shifted(dev_bf16(x), w, oy, ox, T=dev_bf16(T), z_save=zs)
    want = O.wbmm_forward_shifted(x.astype(np.float64), w, oy, ox, T=T)
    assert_bf16(host(y.float()), want, "y")
    if zsave:
        assert torch.equal(zs, y)


@pytest.mark.parametrize("B,C,H,W,w,oy,ox", SHIFT_CASES)
@pytest.mark.parametrize("mix", [False, True])
@pytest.mark.parametrize("src", ["T", "M"])
def test_backward_shifted(B, C, H, W, w, oy, ox, mix, src):
    """dx, dT (and dWmix) on the interleaved grid against the oracle, from the table or from a
    cached matrix (dT is then the gradient of the table M was gathered from); run twice,
    bitwise equal."""
    say(f"backward shifted B={B} C={C} H={H} W={W} w={w} o=({oy},{ox}) mix={mix} src={src}")
    x = synth.normal_f32((B, C, H, W), 1.0, seed=250)
    T = synth.normal_f32((C, 2 * w - 1, 2 * w - 1), 0.05, seed=251)
    dy = synth.normal_f32((B, C, H, W), 1.0, seed=252)
    Wm = synth.normal_f32((C, 3, 3), 0.1, seed=253) if mix else None
    xd, Td, dyd = dev(x), dev(T), dev(dy)
    kw = {"T": Td} if src == "T" else {"M": R().wbmm_build_matrix(Td, w)}
    Wd = dev(Wm) if mix else None
    zs = None
    if mix:
        zs = torch.empty_like(xd)
        R().wbmm_forward_shifted(xd, w, oy, ox, mix_w=Wd, z_save=zs, **kw)
    dx, dT, dW = R().wbmm_backward_shifted(xd, dyd, w, oy, ox, mix_w=Wd, z_saved=zs, **kw)
    z64 = host(zs).astype(np.float64) if mix else None
    wdx, wdT, wdW = O.layer_backward_shifted(x.astype(np.float64), dy.astype(np.float64), w, oy,
                                             ox, T=T, Wmix=Wm, z=z64)
    assert_f32(host(dx), wdx, "dx")
    assert_f32(host(dT), wdT, "dT")
    if mix:
        assert_f32(host(dW), wdW, "dWmix")
    dx2, dT2, _ = R().wbmm_backward_shifted(xd, dyd, w, oy, ox, mix_w=Wd, z_saved=zs, **kw)
    assert torch.equal(dx, dx2) and torch.equal(dT, dT2)


@pytest.mark.parametrize("B,C,H,oy,ox", [(4, 150, 28, 7, 7), (17, 40, 28, 7, 0),
                                         (33, 24, 28, 0, 7), (3, 40, 56, 7, 7),
                                         (17, 16, 56, 0, 7), (70, 16, 14, 7, 7)])
def test_backward_shifted_roll_dx_bitwise_all_channels(B, C, H, oy, ox):
    """One-hot tables on the rolled map (offsets 0 or 7, 14x14 to 56x56): dX = M^T G is G shifted
    back inside each window of the offset grid, bit for bit, in every channel, so the masked
    transposed product drops every pair across pieces and the stores go back through the roll."""
    w = 14
    say(f"backward shifted roll dx shift all channels B={B} C={C} H={H} o=({oy},{ox})")
    x = synth.normal_f32((B, C, H, H), 1.0, seed=43)
    g = synth.normal_f32((B, C, H, H), 1.0, seed=44)
    L1 = 2 * w - 1
    dy = (np.arange(C) * 7 + 1) % L1 - (w - 1)
    dx = (np.arange(C) * 3 + 5) % L1 - (w - 1)
    T = np.zeros((C, L1, L1), np.float32)
    T[np.arange(C), dy + w - 1, dx + w - 1] = 1.0
    got, _, _ = R().wbmm_backward_shifted(dev(x), dev(g), w, oy, ox, T=dev(T), dT=False)
    assert np.array_equal(host(got), _window_shift_grid(g, w, oy, ox, -dy, -dx))


@pytest.mark.parametrize("H", [14, 28, 56])
def test_backward_shifted_roll_partial_outputs(H):
    """The rolled-map backward with only dx or only dT: the other stays unwritten, the one asked
    for matches the oracle."""
    B, C, W, w, o = 5, 3, H, 14, 7
    say(f"backward shifted roll partial outputs H={H}")
    x = synth.normal_f32((B, C, H, W), 1.0, seed=255)
    T = synth.normal_f32((C, 2 * w - 1, 2 * w - 1), 0.05, seed=256)
    dy = synth.normal_f32((B, C, H, W), 1.0, seed=257)
    xd, Td, dyd = dev(x), dev(T), dev(dy)
    wdx, wdT, _ = O.layer_backward_shifted(x.astype(np.float64), dy.astype(np.float64), w, o, o,
                                           T=T)
    dx, dT, _ = R().wbmm_backward_shifted(xd, dyd, w, o, o, T=Td, dT=False)
    assert dT is None
    assert_f32(host(dx), wdx, "dx")
    dx, dT, _ = R().wbmm_backward_shifted(xd, dyd, w, o, o, T=Td, dx=False)
    assert dx is None
    assert_f32(host(dT), wdT, "dT")


def test_shifted_step_full_size_sampled_channels():
    """The interleaved training step at its full size (B=64, C=192, 28x28, w=14, offset (7, 7),
    mix) in the launch configuration the benchmark times: y, z, dx, dT and dWmix of sampled
    channels against the oracle run on those channels alone (the product and the mix act on each
    channel by itself)."""
    B, C, H, W, w, o = 64, 192, 28, 28, 14, 7
    say("shifted step full size")
    x = synth.normal_f32((B, C, H, W), 1.0, seed=260)
    T = synth.normal_f32((C, 2 * w - 1, 2 * w - 1), 0.05, seed=261)
    dy = synth.normal_f32((B, C, H, W), 1.0, seed=262)
    Wm = synth.normal_f32((C, 3, 3), 0.1, seed=263)
    xd, Td, dyd, Wd = dev(x), dev(T), dev(dy), dev(Wm)
    zs = torch.empty_like(xd)
    y = R().wbmm_forward_shifted(xd, w, o, o, T=Td, mix_w=Wd, z_save=zs)
    dx, dT, dW = R().wbmm_backward_shifted(xd, dyd, w, o, o, T=Td, mix_w=Wd, z_saved=zs)
    y, zs, dx, dT, dW = host(y), host(zs), host(dx), host(dT), host(dW)
    for c in (0, 77, 191):
        xc = x[:, c:c + 1].astype(np.float64)
        wy, wz = O.layer_forward_shifted(xc, w, o, o, T=T[c:c + 1], Wmix=Wm[c:c + 1])
        assert_f32(y[:, c:c + 1], wy, f"y c={c}")
        assert_f32(zs[:, c:c + 1], wz, f"z c={c}")
        wdx, wdT, wdW = O.layer_backward_shifted(xc, dy[:, c:c + 1].astype(np.float64), w, o, o,
                                                 T=T[c:c + 1], Wmix=Wm[c:c + 1],
                                                 z=zs[:, c:c + 1].astype(np.float64))
        assert_f32(dx[:, c:c + 1], wdx, f"dx c={c}")
        assert_f32(dT[c:c + 1], wdT, f"dT c={c}")
        assert_f32(dW[c:c + 1], wdW, f"dWmix c={c}")


def test_shifted_zero_offset_is_the_plain_call():
    """(0, 0) through the shifted entry points is the plain call, bit for bit."""
    B, C, H, W, w = 4, 3, 28, 28, 14
    say("shifted zero offset")
    x = dev(synth.normal_f32((B, C, H, W), 1.0, seed=260))
    T = dev(synth.normal_f32((C, 27, 27), 0.05, seed=261))
    dy = dev(synth.normal_f32((B, C, H, W), 1.0, seed=262))
    assert torch.equal(R().wbmm_forward_shifted(x, w, 0, 0, T=T), R().wbmm_forward(x, w, T=T))
    a = R().wbmm_backward_shifted(x, dy, w, 0, 0, T=T)
    b = R().wbmm_backward(x, dy, w, T=T)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_probe_mfma_runs():
    """The matrix-core peak probe (a measurement aid) runs for both operand types and writes
    finite sums."""
    say("probe mfma")
    out = torch.zeros(8 * 256, device="cuda")
    for dt in (torch.float32, torch.bfloat16):
        flops = R().wbmm_probe_mfma(dt, 8, 256, out=out)
        torch.cuda.synchronize()
        o = host(out)
        assert flops > 0 and np.isfinite(o).all() and np.abs(o).max() > 0


# ----------------------------------------------------------------------------- bf16 backward
@pytest.mark.parametrize("B,C,H", [(5, 3, 28), (18, 2, 28), (3, 2, 56), (6, 3, 56)])
@pytest.mark.parametrize("mix", [False, True])
def test_backward_bf16(B, C, H, mix):
    """bf16 maps and table (mixed-precision training) against the oracle on the same bf16 values:
    dx (bf16) and, with a mix, dT within the bf16 bar (G is kept as a bf16 map); without a mix G
    is dy itself, every product is exact and dT meets the fp32 bar; dWmix (fp64 sums of bf16
    values) meets the fp32 bar. Ragged batches leave units part empty; run twice, bitwise."""
    w = 14
    say(f"backward bf16 B={B} C={C} H=W={H} mix={mix}")
    x = synth.round_to_bf16(synth.normal_f32((B, C, H, H), 1.0, seed=270))
    T = synth.round_to_bf16(synth.normal_f32((C, 27, 27), 0.02, seed=271))
    dy = synth.round_to_bf16(synth.normal_f32((B, C, H, H), 1.0, seed=272))
    Wm = synth.normal_f32((C, 3, 3), 0.1, seed=273) if mix else None
    z = (synth.round_to_bf16(O.wbmm_forward(x.astype(np.float64), w, T=T).astype(np.float32))
         if mix else None)
    xd, Td, dyd = dev_bf16(x), dev_bf16(T), dev_bf16(dy)
    zd = dev_bf16(z) if mix else None
    Wd = dev(Wm) if mix else None
    dx, dT, dW = R().wbmm_backward_bf16(xd, dyd, w, Td, mix_w=Wd, z_saved=zd)
    wdx, wdT, wdW = O.layer_backward(x.astype(np.float64), dy.astype(np.float64), w, T=T, Wmix=Wm,
                                     z=z.astype(np.float64) if mix else None)
    assert_bf16(host(dx.float()), wdx, "dx")
    if mix:
        assert_bf16(host(dT), wdT, "dT")
        assert_f32(host(dW), wdW, "dWmix")
    else:
        assert_f32(host(dT), wdT, "dT")
    dx2, dT2, _ = R().wbmm_backward_bf16(xd, dyd, w, Td, mix_w=Wd, z_saved=zd)
    assert torch.equal(dx, dx2) and torch.equal(dT, dT2)


@pytest.mark.parametrize("B,C,H,W,w,layout,mix", [
    (2, 3, 30, 25, 14, "NCHW", True),    # ragged map, image mode (mix adjoint fused)
    (3, 2, 21, 14, 7, "NCHW", False),
    (2, 3, 28, 28, 14, "NHWC", True),    # channels-last
    (1, 2, 56, 56, 7, "NCHW", True),
    (2, 2, 17, 23, 5, "NHWC", False),
    (1, 2, 32, 32, 16, "NCHW", True),
    (2, 2, 128, 128, 14, "NCHW", True),  # window mode: plane-staged mix adjoint (bf16 G)
    (1, 2, 100, 100, 14, "NHWC", True),  # window mode, channels-last: per-pixel mix passes
    # windows wider than 16: dx through the bf16 forward with the rotated table (the fast bf16
    # w = 28 kernel on 56x56 maps), dT on 32x32 row-pair tiles
    (2, 2, 56, 56, 28, "NCHW", True), (1, 2, 40, 37, 20, "NCHW", False),
    (2, 2, 34, 30, 17, "NHWC", True),
])
def test_backward_bf16_general(B, C, H, W, w, layout, mix):
    """bf16 maps and table on the shapes the fast bf16 backward does not cover (any w <= 16,
    ragged maps, NHWC): the general kernels widen bf16 to fp32 tiles exactly. dx within the
    bf16 bar; dT within the fp32 bar without a mix (G = dy, exact products), the bf16 bar with
    one (G may be rounded to bf16); dWmix within the fp32 bar."""
    say(f"backward bf16 general B={B} C={C} H={H} W={W} w={w} {layout} mix={mix}")
    x = synth.round_to_bf16(synth.normal_f32((B, C, H, W), 1.0, seed=275))
    T = synth.round_to_bf16(synth.normal_f32((C, 2 * w - 1, 2 * w - 1), 0.02, seed=276))
    dy = synth.round_to_bf16(synth.normal_f32((B, C, H, W), 1.0, seed=277))
    Wm = synth.normal_f32((C, 3, 3), 0.1, seed=278) if mix else None
    z = (synth.round_to_bf16(O.wbmm_forward(x.astype(np.float64), w, T=T).astype(np.float32))
         if mix else None)
    tl = (lambda a: a) if layout == "NCHW" else (lambda a: np.ascontiguousarray(a.transpose(0, 2, 3, 1)))
    fl = (lambda a: a) if layout == "NCHW" else (lambda a: a.transpose(0, 3, 1, 2))
    xd, Td, dyd = dev_bf16(tl(x)), dev_bf16(T), dev_bf16(tl(dy))
    zd = dev_bf16(tl(z)) if mix else None
    Wd = dev(Wm) if mix else None
    dx, dT, dW = R().wbmm_backward_bf16(xd, dyd, w, Td, mix_w=Wd, z_saved=zd, layout=layout)
    wdx, wdT, wdW = O.layer_backward(x.astype(np.float64), dy.astype(np.float64), w, T=T, Wmix=Wm,
                                     z=z.astype(np.float64) if mix else None)
    assert_bf16(fl(host(dx.float())), wdx, "dx")
    if mix:
        assert_bf16(host(dT), wdT, "dT")
        assert_f32(host(dW), wdW, "dWmix")
    else:
        assert_f32(host(dT), wdT, "dT")
    dx2, dT2, _ = R().wbmm_backward_bf16(xd, dyd, w, Td, mix_w=Wd, z_saved=zd, layout=layout)
    assert torch.equal(dx, dx2) and torch.equal(dT, dT2)


def test_backward_bf16_partial_outputs():
    """Only dT, or only dx: the skipped outputs are not written and the others match."""
    B, C, H, w = 4, 2, 28, 14
    say("backward bf16 partial outputs")
    x = synth.round_to_bf16(synth.normal_f32((B, C, H, H), 1.0, seed=280))
    T = synth.round_to_bf16(synth.normal_f32((C, 27, 27), 0.02, seed=281))
    dy = synth.round_to_bf16(synth.normal_f32((B, C, H, H), 1.0, seed=282))
    xd, Td, dyd = dev_bf16(x), dev_bf16(T), dev_bf16(dy)
    dx0, dT, _ = R().wbmm_backward_bf16(xd, dyd, w, Td, dx=False)
    assert dx0 is None
    dx, dT0, _ = R().wbmm_backward_bf16(xd, dyd, w, Td, dT=False)
    assert dT0 is None
    wdx, wdT, _ = O.layer_backward(x.astype(np.float64), dy.astype(np.float64), w, T=T)
    assert_f32(host(dT), wdT, "dT")
    assert_bf16(host(dx.float()), wdx, "dx")


@pytest.mark.parametrize("B,C,H,W,w", [(4, 3, 28, 28, 14), (2, 2, 128, 128, 14), (3, 2, 20, 17, 6),
                                       (5, 2, 56, 56, 14), (3, 2, 56, 56, 7), (2, 2, 56, 56, 28)])
@pytest.mark.parametrize("zsave", [True, False])
def test_forward_bf16_with_mix(B, C, H, W, w, zsave):
    """bf16 maps with the 3x3 mix: y and z_save in bf16, against the oracle on bf16 values. Fast
    bf16 shapes run the fast forward into z (z_save or the workspace) and a plane-staged mix pass;
    the general kernel fuses the mix in image mode and runs it as a pass in window mode."""
    say(f"forward bf16 mix B={B} C={C} H={H} W={W} w={w} zsave={zsave}")
    x = synth.round_to_bf16(synth.normal_f32((B, C, H, W), 1.0, seed=290))
    T = synth.round_to_bf16(synth.normal_f32((C, 2 * w - 1, 2 * w - 1), 0.02, seed=291))
    Wm = synth.normal_f32((C, 3, 3), 0.1, seed=292)
    zs = torch.empty((B, C, H, W), dtype=torch.bfloat16, device="cuda") if zsave else None
    y = R().wbmm_forward(dev_bf16(x), w, T=dev_bf16(T), mix_w=dev(Wm), z_save=zs)
    want_y, want_z = O.layer_forward(x.astype(np.float64), w, T=T, Wmix=Wm)
    assert y.dtype == torch.bfloat16
    assert_bf16(host(y.float()), want_y, "y")
    if zsave:
        assert_bf16(host(zs.float()), want_z, "z")


def test_bf16_training_step_with_mix():
    """A bf16 layer training step with the mix: the bf16 forward's z_save feeds the bf16
    backward; all gradients against the oracle on the same bf16 values."""
    B, C, H, w = 8, 3, 28, 14
    say("bf16 training step with mix")
    x = synth.round_to_bf16(synth.normal_f32((B, C, H, H), 1.0, seed=300))
    T = synth.round_to_bf16(synth.normal_f32((C, 27, 27), 0.02, seed=301))
    Wm = synth.normal_f32((C, 3, 3), 0.1, seed=302)
    dy = synth.round_to_bf16(synth.normal_f32((B, C, H, H), 1.0, seed=303))
    xd, Td, Wd = dev_bf16(x), dev_bf16(T), dev(Wm)
    zs = torch.empty((B, C, H, H), dtype=torch.bfloat16, device="cuda")
    R().wbmm_forward(xd, w, T=Td, mix_w=Wd, z_save=zs)
    dx, dT, dW = R().wbmm_backward_bf16(xd, dev_bf16(dy), w, Td, mix_w=Wd, z_saved=zs)
    z = host(zs.float()).astype(np.float64)
    wdx, wdT, wdW = O.layer_backward(x.astype(np.float64), dy.astype(np.float64), w, T=T,
                                     Wmix=Wm, z=z)
    assert_bf16(host(dx.float()), wdx, "dx")
    assert_bf16(host(dT), wdT, "dT")
    assert_f32(host(dW), wdW, "dWmix")


@pytest.mark.parametrize("kind", ["hier", "shift"])
def test_nhwc_hier_and_shifted(kind):
    """Channels-last maps through the on-chip fold and the interleaved grid (general kernels):
    forward with the mix and backward, against the oracle on the transposed maps."""
    B, C, H, W, w = 2, 3, 28, 28, 14
    say(f"nhwc {kind}")
    x = synth.normal_f32((B, C, H, W), 1.0, seed=310)
    T = synth.normal_f32((C, 27, 27), 0.05, seed=311)
    Ts = synth.normal_f32((C, 13, 13), 0.05, seed=312)
    Wm = synth.normal_f32((C, 3, 3), 0.1, seed=313)
    dy = synth.normal_f32((B, C, H, W), 1.0, seed=314)
    nhwc = lambda a: dev(np.ascontiguousarray(a.transpose(0, 2, 3, 1)))
    back = lambda t: host(t).transpose(0, 3, 1, 2)
    xd, dyd, Td, Wd = nhwc(x), nhwc(dy), dev(T), dev(Wm)
    zs = torch.empty_like(xd)
    if kind == "hier":
        y = R().wbmm_forward_hier(xd, w, 7, Td, dev(Ts), mix_w=Wd, layout="NHWC", z_save=zs)
        dx, dT, dTs, dW = R().wbmm_backward_hier(xd, dyd, w, 7, Td, dev(Ts), mix_w=Wd, z_saved=zs,
                                                 layout="NHWC")
        wy, wz = O.layer_forward_hier(x.astype(np.float64), w, 7, T, Ts, Wmix=Wm)
        wdx, wdT, wdTs, wdW = O.layer_backward_hier(x.astype(np.float64), dy.astype(np.float64),
                                                    w, 7, T, Ts, Wmix=Wm,
                                                    z=back(zs).astype(np.float64))
        assert_f32(host(dTs), wdTs, "dT_sub")
    else:
        y = R().wbmm_forward_shifted(xd, w, 7, 7, T=Td, mix_w=Wd, layout="NHWC", z_save=zs)
        dx, dT, dW = R().wbmm_backward_shifted(xd, dyd, w, 7, 7, T=Td, mix_w=Wd, z_saved=zs,
                                               layout="NHWC")
        wy, wz = O.layer_forward_shifted(x.astype(np.float64), w, 7, 7, T=T, Wmix=Wm)
        wdx, wdT, wdW = O.layer_backward_shifted(x.astype(np.float64), dy.astype(np.float64), w,
                                                 7, 7, T=T, Wmix=Wm,
                                                 z=back(zs).astype(np.float64))
    assert_f32(back(y), wy, "y")
    assert_f32(back(zs), wz, "z")
    assert_f32(back(dx), wdx, "dx")
    assert_f32(host(dT), wdT, "dT")
    assert_f32(host(dW), wdW, "dWmix")
