"""Pins for the CPU oracle: it is checked against things other than itself.

Each test ties an oracle function to something the pages or the mathematics fix:
  * a hand-worked index table (tests/golden/index_w2.txt) and the exact pair-count invariant;
  * a brute-force per-output sum over window positions (no matrices, no index table);
  * the per-window closed form: WBMM equals a zero-padded (2w-1)x(2w-1) depthwise correlation of
    each window with the 180-degree rotated table, computed with torch's conv2d (CPU, float64)
    and with a numpy shift-and-add;
  * exact special cases: one-hot tables give the identity / windowed shifts, all-ones data counts
    real pixels per window, the dT of all-ones data counts pairs per offset;
  * the adjoint identity, torch autograd of the closed form, and finite differences for the
    backward;
  * torch's conv2d for the 3x3 depthwise mix and its gradients;
  * for the k x k depthwise convolution (the pages' DW-Std baseline): torch's conv2d, a pure-loop
    brute force, one-hot kernels as exact shifts, and its two exact relations to the rest of the
    oracle (k = 3 is the 3x3 mix; on a single-window image with k = 2w-1 it is WBMM).
A plausible slip in the oracle (a flipped sign, a transposed matrix, a dropped term, a wrong
crop/pad) fails at least one of these.
"""
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import wbmm_oracle as O
from receptive_field_spatial_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(shape, sigma=1.0, seed=0):
    return synth.normal_f32(shape, sigma, seed).astype(np.float64)


# ----------------------------------------------------------------------------- brute force
def brute_force(x, T, w):
    """Per-output sum over the positions of the output's own window (pure Python loops)."""
    B, C, H, W = x.shape
    out = np.zeros((B, C, H, W))
    for b in range(B):
        for c in range(C):
            for py in range(H):
                for px in range(W):
                    wy0, wx0 = (py // w) * w, (px // w) * w
                    acc = 0.0
                    for qy in range(wy0, min(wy0 + w, H)):
                        for qx in range(wx0, min(wx0 + w, W)):
                            acc += T[c, py - qy + w - 1, px - qx + w - 1] * x[b, c, qy, qx]
                    out[b, c, py, px] = acc
    return out


def windows_of(x, w):
    """(B, C, Hp, Wp) padded map -> (B*nH*nW, C, w, w) stack of windows."""
    B, C, Hp, Wp = x.shape
    nH, nW = Hp // w, Wp // w
    return x.reshape(B, C, nH, w, nW, w).transpose(0, 2, 4, 1, 3, 5).reshape(-1, C, w, w)


def unwindows(t, B, Hp, Wp, w):
    C = t.shape[1]
    nH, nW = Hp // w, Wp // w
    return t.reshape(B, nH, nW, C, w, w).transpose(0, 3, 1, 4, 2, 5).reshape(B, C, Hp, Wp)


def closed_form_torch(x, T, w):
    """Per-window depthwise correlation with rot180(T), zero padding w-1, via torch conv2d."""
    B, C, H, W = x.shape
    Hp, Wp = O.padded_hw(H, W, w)
    xp = np.zeros((B, C, Hp, Wp))
    xp[:, :, :H, :W] = x
    win = torch.from_numpy(windows_of(xp, w))
    kern = torch.from_numpy(np.ascontiguousarray(T[:, ::-1, ::-1]))[:, None]
    out = F.conv2d(win, kern, padding=w - 1, groups=C).numpy()
    return unwindows(out, B, Hp, Wp, w)[:, :, :H, :W]


def closed_form_shift_add(x, T, w):
    """Same closed form as a numpy shift-and-add over the (2w-1)^2 offsets inside each window."""
    B, C, H, W = x.shape
    Hp, Wp = O.padded_hw(H, W, w)
    xp = np.zeros((B, C, Hp, Wp))
    xp[:, :, :H, :W] = x
    win = windows_of(xp, w)
    out = np.zeros_like(win)
    for dy in range(-(w - 1), w):
        for dx in range(-(w - 1), w):
            # out[y, x] += T[dy + w - 1, dx + w - 1] * in[y - dy, x - dx]
            ys, yd = (slice(0, w - dy), slice(dy, w)) if dy >= 0 else (slice(-dy, w), slice(0, w + dy))
            xs, xd = (slice(0, w - dx), slice(dx, w)) if dx >= 0 else (slice(-dx, w), slice(0, w + dx))
            out[:, :, yd, xd] += T[None, :, dy + w - 1, dx + w - 1, None, None] * win[:, :, ys, xs]
    return unwindows(out, B, Hp, Wp, w)[:, :, :H, :W]


# ----------------------------------------------------------------------------- index / matrix
def test_index_hand_worked_w2():
    want = np.loadtxt(os.path.join(GOLDEN, "index_w2.txt"), dtype=np.int64)
    got = O.build_index(2)
    assert got.dtype == np.int32
    assert np.array_equal(got, want)


def test_index_w1_is_single_entry():
    assert np.array_equal(O.build_index(1), np.array([[0]], dtype=np.int32))


@pytest.mark.parametrize("w", [1, 2, 3, 4, 7, 14, 28])
def test_index_pair_counts(w):
    """Offset (dy, dx) occurs (w-|dy|)(w-|dx|) times among the d*d pairs; all in range."""
    idx = O.build_index(w)
    L = (2 * w - 1) ** 2
    assert idx.min() >= 0 and idx.max() < L
    counts = np.bincount(idx.ravel(), minlength=L).reshape(2 * w - 1, 2 * w - 1)
    run = w - np.abs(np.arange(-(w - 1), w))
    assert np.array_equal(counts, np.outer(run, run))
    assert counts.sum() == w ** 4


@pytest.mark.parametrize("w", [3, 7, 14])
def test_matrix_structure(w):
    C = 3
    T = rnd((C, 2 * w - 1, 2 * w - 1), seed=1).astype(np.float32)
    M = O.build_matrix(T, w)
    assert M.dtype == np.float32 and M.shape == (C, w * w, w * w)
    # diagonal = table centre
    for c in range(C):
        assert np.all(np.diag(M[c]) == T[c, w - 1, w - 1])
    # entry depends only on the position difference (block-Toeplitz with Toeplitz blocks)
    y, x = np.divmod(np.arange(w * w), w)
    for c in range(C):
        for i in range(0, w * w, max(1, w * w // 7)):
            for j in range(0, w * w, max(1, w * w // 5)):
                assert M[c, i, j] == T[c, y[i] - y[j] + w - 1, x[i] - x[j] + w - 1]
    # rotating the table by 180 degrees transposes every M_c exactly
    Mr = O.build_matrix(np.ascontiguousarray(T[:, ::-1, ::-1]), w)
    assert np.array_equal(Mr, M.transpose(0, 2, 1))


# ----------------------------------------------------------------------------- forward
def test_forward_brute_force_tiny_workload():
    wl = synth.WORKLOADS["tiny_w7"]
    inp = synth.draw_inputs(wl)
    x, T = inp["x"].astype(np.float64), inp["T"].astype(np.float64)
    got = O.wbmm_forward(x, wl.w, T=T)
    want = brute_force(x, T, wl.w)
    assert np.allclose(got, want, rtol=0, atol=1e-13)


@pytest.mark.parametrize("B,C,H,W,w", [(2, 3, 10, 13, 4), (1, 2, 5, 5, 5), (1, 2, 7, 3, 3),
                                       (2, 1, 4, 4, 1)])
def test_forward_brute_force_ragged(B, C, H, W, w):
    x = rnd((B, C, H, W), seed=2)
    T = rnd((C, 2 * w - 1, 2 * w - 1), 0.5, seed=3)
    got = O.wbmm_forward(x, w, T=T)
    assert got.shape == (B, C, H, W)
    assert np.allclose(got, brute_force(x, T, w), rtol=0, atol=1e-12)


@pytest.mark.parametrize("B,C,H,W,w", [(1, 8, 28, 28, 7), (2, 3, 28, 28, 14), (1, 2, 30, 17, 6),
                                       (1, 2, 56, 56, 28)])
def test_forward_closed_form(B, C, H, W, w):
    x = rnd((B, C, H, W), seed=4)
    T = rnd((C, 2 * w - 1, 2 * w - 1), 0.02, seed=5)
    got = O.wbmm_forward(x, w, T=T)
    ref_t = closed_form_torch(x, T, w)
    ref_n = closed_form_shift_add(x, T, w)
    scale = np.abs(ref_t).max()
    assert np.abs(got - ref_t).max() <= 1e-12 * scale
    assert np.abs(got - ref_n).max() <= 1e-12 * scale


def test_forward_unrotated_kernel_is_not_it():
    """Sanity of the orientation pin: the unrotated table gives a visibly different result."""
    w = 4
    x = rnd((1, 2, 8, 8), seed=6)
    T = rnd((2, 7, 7), seed=7)
    got = O.wbmm_forward(x, w, T=T)
    wrong = closed_form_torch(x, np.ascontiguousarray(T[:, ::-1, ::-1]), w)
    assert np.abs(got - wrong).max() > 1e-2


@pytest.mark.parametrize("w", [1, 3, 7])
def test_one_hot_centre_is_identity(w):
    x = rnd((2, 2, 2 * w + 1, 3 * w - 1), seed=8)
    T = np.zeros((2, 2 * w - 1, 2 * w - 1))
    T[:, w - 1, w - 1] = 1.0
    assert np.array_equal(O.wbmm_forward(x, w, T=T), x)


@pytest.mark.parametrize("a,b", [(1, 0), (0, 1), (-2, 1), (3, -3), (-4, -4)])
def test_one_hot_offset_is_windowed_shift(a, b):
    """T one-hot at offset (a, b): out(y, x) = in(y - a, x - b) inside the window, else 0."""
    w = 5
    B, C, H, W = 1, 2, 10, 15
    x = rnd((B, C, H, W), seed=9)
    T = np.zeros((C, 2 * w - 1, 2 * w - 1))
    T[:, a + w - 1, b + w - 1] = 1.0
    got = O.wbmm_forward(x, w, T=T)
    want = np.zeros_like(x)
    for py in range(H):
        for px in range(W):
            qy, qx = py - a, px - b
            if (0 <= qy < H and 0 <= qx < W and qy // w == py // w and qx // w == px // w):
                want[:, :, py, px] = x[:, :, qy, qx]
    assert np.array_equal(got, want)


def test_ones_count_real_pixels_per_window():
    """x = 1 and T = 1: each output equals the number of unpadded pixels in its window."""
    w = 4
    H, W = 10, 13
    x = np.ones((1, 1, H, W))
    T = np.ones((1, 2 * w - 1, 2 * w - 1))
    got = O.wbmm_forward(x, w, T=T)
    for py in range(H):
        for px in range(W):
            rows = min(w, H - (py // w) * w)
            cols = min(w, W - (px // w) * w)
            assert got[0, 0, py, px] == rows * cols


def test_forward_linearity():
    w = 4
    x1, x2 = rnd((1, 2, 8, 12), seed=10), rnd((1, 2, 8, 12), seed=11)
    T1, T2 = rnd((2, 7, 7), seed=12), rnd((2, 7, 7), seed=13)
    f = O.wbmm_forward
    assert np.allclose(f(2 * x1 - 3 * x2, w, T=T1), 2 * f(x1, w, T=T1) - 3 * f(x2, w, T=T1), atol=1e-12)
    assert np.allclose(f(x1, w, T=0.5 * T1 + T2), 0.5 * f(x1, w, T=T1) + f(x1, w, T=T2), atol=1e-12)


def test_cached_matrix_path_matches_table_path():
    w = 7
    x = rnd((2, 3, 14, 21), seed=14)
    T = rnd((3, 13, 13), seed=15)
    M = O.build_matrix(T, w)
    assert np.array_equal(O.wbmm_forward(x, w, M=M), O.wbmm_forward(x, w, T=T))


# ----------------------------------------------------------------------------- fold
def test_fold_identity_two_window_sizes():
    """Folding T_sub into M equals adding a separate s-window WBMM of the same padded map."""
    w, s = 14, 7
    x = rnd((2, 3, 28, 30), seed=16)
    T = rnd((3, 27, 27), 0.02, seed=17).astype(np.float32)
    Ts = rnd((3, 13, 13), 0.02, seed=18).astype(np.float32)
    Mf = O.fold_hier(O.build_matrix(T, w), Ts, w, s)
    got = O.wbmm_forward(x, w, M=Mf)
    # s-window WBMM on the w-padded map, then crop
    Hp, Wp = O.padded_hw(28, 30, w)
    xp = np.zeros((2, 3, Hp, Wp))
    xp[:, :, :28, :30] = x
    want = (O.wbmm_forward(x, w, T=T.astype(np.float64))
            + O.wbmm_forward(xp, s, T=Ts.astype(np.float64))[:, :, :28, :30])
    # the fold adds in float32, so compare at float32 resolution of M
    assert np.abs(got - want).max() <= 1e-6


def test_fold_touches_only_same_subwindow_pairs():
    w, s = 14, 7
    T = rnd((2, 27, 27), 0.02, seed=19).astype(np.float32)
    Ts = rnd((2, 13, 13), 0.02, seed=20).astype(np.float32)
    M = O.build_matrix(T, w)
    Mf = O.fold_hier(M, Ts, w, s)
    assert Mf.dtype == np.float32
    y, x = np.divmod(np.arange(w * w), w)
    n_changed_pairs = 0
    for i in range(w * w):
        for j in range(w * w):
            same = (y[i] // s == y[j] // s) and (x[i] // s == x[j] // s)
            if same:
                n_changed_pairs += 1
                add = Ts[:, y[i] % s - y[j] % s + s - 1, x[i] % s - x[j] % s + s - 1]
                assert np.array_equal(Mf[:, i, j], (M[:, i, j] + add).astype(np.float32))
            else:
                assert np.array_equal(Mf[:, i, j], M[:, i, j])
    assert n_changed_pairs == 4 * 49 * 49  # 4 sub-windows of 49 pixels each


# ----------------------------------------------------------------------------- mix
def test_mix_forward_matches_torch_conv2d():
    z = rnd((2, 5, 9, 11), seed=21)
    Wm = rnd((5, 3, 3), 0.1, seed=22)
    want = F.conv2d(torch.from_numpy(z), torch.from_numpy(Wm)[:, None], padding=1, groups=5).numpy()
    assert np.allclose(O.mix_forward(z, Wm), want, rtol=0, atol=1e-14)


def test_mix_backward_matches_torch_autograd():
    z = torch.from_numpy(rnd((2, 5, 9, 11), seed=23)).requires_grad_(True)
    Wm = torch.from_numpy(rnd((5, 3, 3), 0.1, seed=24)).requires_grad_(True)
    dy = rnd((2, 5, 9, 11), seed=25)
    y = F.conv2d(z, Wm[:, None], padding=1, groups=5)
    y.backward(torch.from_numpy(dy))
    dz, dW = O.mix_backward(dy, z.detach().numpy(), Wm.detach().numpy())
    assert np.allclose(dz, z.grad.numpy(), rtol=0, atol=1e-13)
    assert np.allclose(dW, Wm.grad.numpy(), rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- backward
def test_dx_adjoint_identity():
    w = 5
    x = rnd((2, 3, 12, 9), seed=26)
    g = rnd((2, 3, 12, 9), seed=27)
    T = rnd((3, 9, 9), seed=28)
    dx, _ = O.wbmm_backward(x, g, w, T=T)
    lhs = np.sum(O.wbmm_forward(x, w, T=T) * g)
    rhs = np.sum(x * dx)
    assert abs(lhs - rhs) <= 1e-12 * abs(lhs) + 1e-12


def test_backward_matches_torch_autograd_of_closed_form():
    """dx and dT against autograd through the per-window conv2d route (independent of the matrix form)."""
    w = 4
    B, C, H, W = 2, 3, 10, 9
    x_np = rnd((B, C, H, W), seed=29)
    T_np = rnd((C, 7, 7), seed=30)
    g = rnd((B, C, H, W), seed=31)
    Hp, Wp = O.padded_hw(H, W, w)
    x = torch.from_numpy(x_np).requires_grad_(True)
    T = torch.from_numpy(T_np).requires_grad_(True)
    xp = F.pad(x, (0, Wp - W, 0, Hp - H))
    nH, nW = Hp // w, Wp // w
    win = xp.reshape(B, C, nH, w, nW, w).permute(0, 2, 4, 1, 3, 5).reshape(-1, C, w, w)
    out = F.conv2d(win, torch.flip(T, dims=(1, 2))[:, None], padding=w - 1, groups=C)
    y = out.reshape(B, nH, nW, C, w, w).permute(0, 3, 1, 4, 2, 5).reshape(B, C, Hp, Wp)[:, :, :H, :W]
    y.backward(torch.from_numpy(g))
    dx, dT = O.wbmm_backward(x_np, g, w, T=T_np)
    assert np.allclose(dx, x.grad.numpy(), rtol=0, atol=1e-12)
    assert np.allclose(dT, T.grad.numpy(), rtol=0, atol=1e-11)


def test_dT_all_ones_counts_pairs():
    """x = 1, dz = 1, no mix: dT[c, dy, dx] = N * (w-|dy|) * (w-|dx|) exactly."""
    w = 7
    B, C, H, W = 3, 2, 14, 21
    N = B * (H // w) * (W // w)
    x = np.ones((B, C, H, W))
    T = rnd((C, 13, 13), seed=32)
    _, dT = O.wbmm_backward(x, np.ones_like(x), w, T=T)
    run = w - np.abs(np.arange(-(w - 1), w))
    for c in range(C):
        assert np.array_equal(dT[c], N * np.outer(run, run).astype(np.float64))


@pytest.mark.slow
def test_dT_finite_differences_train_slice():
    """Central differences of L(T) = sum(dY * y(T)) on a 1-channel slice of the training workload.

    L is linear in T, so the central difference equals the derivative up to float64 rounding for
    any step; the mix is included.
    """
    wl = synth.WORKLOADS["train_w14"]
    inp = synth.draw_inputs(wl)
    w = wl.w
    x = inp["x"][:, :1].astype(np.float64)
    T = inp["T"][:1].astype(np.float64)
    Wm = inp["Wmix"][:1]
    dY = inp["dY"][:, :1].astype(np.float64)
    _, dT, _ = O.layer_backward(x, dY, w, T=T, Wmix=Wm)
    L0 = (2 * w - 1) ** 2
    h = 1e-2
    fd = np.empty(L0)
    for k in range(L0):
        Tp = T.copy().reshape(-1)
        Tm = T.copy().reshape(-1)
        Tp[k] += h
        Tm[k] -= h
        yp, _ = O.layer_forward(x, w, T=Tp.reshape(T.shape), Wmix=Wm)
        ym, _ = O.layer_forward(x, w, T=Tm.reshape(T.shape), Wmix=Wm)
        fd[k] = (np.sum(dY * yp) - np.sum(dY * ym)) / (2 * h)
    err = np.abs(fd - dT.reshape(-1)).max()
    assert err <= 1e-9 * np.abs(dT).max()


def test_mix_finite_differences():
    z = rnd((1, 2, 6, 7), seed=33)
    Wm = rnd((2, 3, 3), 0.1, seed=34)
    dy = rnd((1, 2, 6, 7), seed=35)
    _, dW = O.mix_backward(dy, z, Wm)
    h = 1e-3
    for c in range(2):
        for u in range(3):
            for t in range(3):
                Wp_, Wn_ = Wm.copy(), Wm.copy()
                Wp_[c, u, t] += h
                Wn_[c, u, t] -= h
                fd = (np.sum(dy * O.mix_forward(z, Wp_)) - np.sum(dy * O.mix_forward(z, Wn_))) / (2 * h)
                assert abs(fd - dW[c, u, t]) <= 1e-10


def test_cached_matrix_backward_matches_table_backward():
    w = 4
    x = rnd((2, 2, 8, 8), seed=36)
    g = rnd((2, 2, 8, 8), seed=37)
    T = rnd((2, 7, 7), seed=38)
    dx1, dT1 = O.wbmm_backward(x, g, w, T=T)
    dx2, dT2 = O.wbmm_backward(x, g, w, M=O.build_matrix(T, w))
    assert np.array_equal(dx1, dx2) and np.array_equal(dT1, dT2)


# ----------------------------------------------------------------------------- hierarchical backward
def hier_brute_force(x, g, T, Ts, w, s):
    """Pure loops over images, windows and pixel pairs: (dx, dT, dT_sub) of the folded layer,
    with the pair weight T[dy][dx] + (same s-sub-window ? T_sub[dy%][dx%] : 0) written out."""
    B, C, H, W = x.shape
    dx = np.zeros_like(x)
    dT = np.zeros_like(T)
    dTs = np.zeros_like(Ts)
    for b in range(B):
        for c in range(C):
            for wy0 in range(0, H, w):
                for wx0 in range(0, W, w):
                    pix = [(py, px) for py in range(wy0, min(wy0 + w, H))
                           for px in range(wx0, min(wx0 + w, W))]
                    for (py, px) in pix:      # output pixel i
                        for (qy, qx) in pix:  # input pixel j
                            yi, xi, yj, xj = py - wy0, px - wx0, qy - wy0, qx - wx0
                            same = yi // s == yj // s and xi // s == xj // s
                            m = T[c, yi - yj + w - 1, xi - xj + w - 1]
                            if same:
                                m += Ts[c, yi % s - yj % s + s - 1, xi % s - xj % s + s - 1]
                            dx[b, c, qy, qx] += m * g[b, c, py, px]
                            gx = g[b, c, py, px] * x[b, c, qy, qx]
                            dT[c, yi - yj + w - 1, xi - xj + w - 1] += gx
                            if same:
                                dTs[c, yi % s - yj % s + s - 1, xi % s - xj % s + s - 1] += gx
    return dx, dT, dTs


@pytest.mark.parametrize("B,C,H,W,w,s", [(2, 2, 8, 8, 4, 2), (1, 2, 10, 7, 4, 2), (1, 1, 6, 6, 6, 3)])
def test_hier_backward_brute_force(B, C, H, W, w, s):
    x = rnd((B, C, H, W), seed=51)
    g = rnd((B, C, H, W), seed=52)
    T = rnd((C, 2 * w - 1, 2 * w - 1), seed=53)
    Ts = rnd((C, 2 * s - 1, 2 * s - 1), seed=54)
    dx, dT, dTs = O.wbmm_backward_hier(x, g, w, s, T, Ts)
    bx, bT, bTs = hier_brute_force(x, g, T, Ts, w, s)
    assert np.allclose(dx, bx, rtol=0, atol=1e-12)
    assert np.allclose(dT, bT, rtol=0, atol=1e-12)
    assert np.allclose(dTs, bTs, rtol=0, atol=1e-12)


def test_hier_finite_differences_with_mix():
    """Central differences of L = sum(dY * y(T, T_sub, x)) through the fold and the mix: exact up to
    rounding, since L is linear in each of T_sub, T and x."""
    w, s = 4, 2
    x = rnd((2, 2, 8, 8), seed=55)
    T = rnd((2, 7, 7), 0.1, seed=56)
    Ts = rnd((2, 3, 3), 0.1, seed=57)
    Wm = rnd((2, 3, 3), 0.1, seed=58)
    dY = rnd((2, 2, 8, 8), seed=59)
    dx, dT, dTs, dW = O.layer_backward_hier(x, dY, w, s, T, Ts, Wmix=Wm)

    def L(x_=x, T_=T, Ts_=Ts):
        return np.sum(dY * O.layer_forward_hier(x_, w, s, T_, Ts_, Wmix=Wm)[0])

    h = 1e-3
    for k in range(Ts.size):
        P, Mn = Ts.copy().reshape(-1), Ts.copy().reshape(-1)
        P[k] += h
        Mn[k] -= h
        fd = (L(Ts_=P.reshape(Ts.shape)) - L(Ts_=Mn.reshape(Ts.shape))) / (2 * h)
        assert abs(fd - dTs.reshape(-1)[k]) <= 1e-9
    for k in (0, 11, 24, 48, 97):
        P, Mn = T.copy().reshape(-1), T.copy().reshape(-1)
        P[k] += h
        Mn[k] -= h
        fd = (L(T_=P.reshape(T.shape)) - L(T_=Mn.reshape(T.shape))) / (2 * h)
        assert abs(fd - dT.reshape(-1)[k]) <= 1e-9
    for k in (0, 37, 64, 255):
        P, Mn = x.copy().reshape(-1), x.copy().reshape(-1)
        P[k] += h
        Mn[k] -= h
        fd = (L(x_=P.reshape(x.shape)) - L(x_=Mn.reshape(x.shape))) / (2 * h)
        assert abs(fd - dx.reshape(-1)[k]) <= 1e-9


def test_hier_zero_sub_table_is_plain_backward():
    """T_sub = 0: dx and dT are exactly the unfolded ones; dT_sub sums the same-sub-window part."""
    w, s = 14, 7
    x = rnd((1, 2, 28, 14), seed=60)
    g = rnd((1, 2, 28, 14), seed=61)
    T = rnd((2, 27, 27), 0.02, seed=62)
    dx, dT, dTs = O.wbmm_backward_hier(x, g, w, s, T, np.zeros((2, 13, 13)))
    dx0, dT0 = O.wbmm_backward(x, g, w, T=T)
    assert np.array_equal(dx, dx0) and np.array_equal(dT, dT0)
    # same-sub-window offsets are the central 13 x 13 of dT: dT_sub is at most that, and every
    # same-sub-window pair is also counted in dT
    assert dTs.shape == (2, 13, 13)
    ones = np.ones_like(x)
    _, dT1, dTs1 = O.wbmm_backward_hier(ones, ones, w, s, T, np.zeros((2, 13, 13)))
    run = s - np.abs(np.arange(-(s - 1), s))
    n_sub = 2 * 4  # windows x sub-windows per window
    for c in range(2):
        assert np.array_equal(dTs1[c], n_sub * np.outer(run, run).astype(np.float64))


# ----------------------------------------------------------------------------- misc pins
def test_receptive_field_ratio():
    """The abstract's 7.8x per-layer receptive field: a 14x14 window covers 196 pixels, a 5x5 kernel 25."""
    assert round((14 * 14) / (5 * 5), 1) == 7.8


def test_bf16_rounding_bits():
    vals = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 1.0 + 2.0 ** -7,
                     1.0 + 2.0 ** -8 + 2.0 ** -20], dtype=np.float32)
    bits = synth.f32_to_bf16_bits(vals)
    # 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 is a tie -> even (1+2^-6);
    # 1+2^-8+2^-20 is above the tie -> rounds up to 1+2^-7.
    assert list(bits) == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x3F81, 0x3F81]
    back = synth.bf16_bits_to_f32(bits)
    assert back[3] == -2.5 and back[2] == np.float32(1.0 + 2 ** -6)


def test_inputs_are_seeded_and_ordered():
    wl = synth.WORKLOADS["tiny_w7"]
    a = synth.draw_inputs(wl, seed=0)
    b = synth.draw_inputs(wl, seed=0)
    assert all(np.array_equal(a[k], b[k]) for k in a)
    rng = np.random.default_rng(0)
    x = (rng.standard_normal((1, 8, 28, 28)) * 1.0).astype(np.float32)
    assert np.array_equal(a["x"], x)
    assert a["T"].shape == (8, 13, 13) and abs(float(a["T"].std()) - 0.02) < 0.004


# ----------------------------------------------------------------------------- DW-Std (k x k)
def dw_brute_force(x, Wd):
    """Per-output sum over the k x k neighbours inside the image (pure Python loops)."""
    B, C, H, W = x.shape
    k = Wd.shape[-1]
    p = k // 2
    out = np.zeros((B, C, H, W))
    for b in range(B):
        for c in range(C):
            for h in range(H):
                for v in range(W):
                    acc = 0.0
                    for u in range(k):
                        for t in range(k):
                            hh, vv = h + u - p, v + t - p
                            if 0 <= hh < H and 0 <= vv < W:
                                acc += Wd[c, u, t] * x[b, c, hh, vv]
                    out[b, c, h, v] = acc
    return out


@pytest.mark.parametrize("k,H,W", [(3, 9, 11), (5, 14, 14), (9, 12, 7), (13, 20, 17), (13, 5, 6)])
def test_dw_conv_matches_torch_conv2d(k, H, W):
    x = rnd((2, 4, H, W), seed=130 + k)
    Wd = rnd((4, k, k), 0.05, seed=131 + k)
    want = F.conv2d(torch.from_numpy(x), torch.from_numpy(Wd)[:, None], padding=k // 2,
                    groups=4).numpy()
    got = O.dw_conv_forward(x, Wd)
    assert np.abs(got - want).max() <= 1e-12 * max(1.0, np.abs(want).max())


@pytest.mark.parametrize("k,H,W", [(5, 7, 6), (7, 9, 9), (13, 6, 15)])
def test_dw_conv_brute_force(k, H, W):
    x = rnd((1, 2, H, W), seed=140 + k)
    Wd = rnd((2, k, k), 0.05, seed=141 + k)
    assert np.allclose(O.dw_conv_forward(x, Wd), dw_brute_force(x, Wd), rtol=0, atol=1e-12)


@pytest.mark.parametrize("k,u,t", [(5, 0, 4), (7, 3, 3), (13, 12, 1), (9, 2, 6)])
def test_dw_conv_one_hot_is_shift(k, u, t):
    """A single 1 at (u, t) copies x shifted by (u - p, t - p), zeros where it leaves the image."""
    x = rnd((2, 3, 16, 18), seed=150)
    Wd = np.zeros((3, k, k))
    Wd[:, u, t] = 1.0
    p = k // 2
    dy, dx = u - p, t - p
    want = np.zeros_like(x)
    H, W = x.shape[2:]
    for h in range(H):
        for v in range(W):
            if 0 <= h + dy < H and 0 <= v + dx < W:
                want[:, :, h, v] = x[:, :, h + dy, v + dx]
    assert np.array_equal(O.dw_conv_forward(x, Wd), want)


def test_dw_conv_k3_is_the_mix():
    z = rnd((2, 5, 9, 13), seed=160)
    Wm = rnd((5, 3, 3), 0.1, seed=161)
    assert np.allclose(O.dw_conv_forward(z, Wm), O.mix_forward(z, Wm), rtol=0, atol=1e-14)


@pytest.mark.parametrize("w", [2, 5, 7])
def test_dw_conv_on_one_window_is_wbmm(w):
    """An image that is exactly one window: WBMM with table T equals DW-Std with k = 2w-1 and the
    180-degree rotated table as its kernel (the zero padding of the convolution stands in for the
    window edge)."""
    x = rnd((3, 4, w, w), seed=170 + w)
    T = rnd((4, 2 * w - 1, 2 * w - 1), 0.05, seed=171 + w)
    dw = O.dw_conv_forward(x, np.ascontiguousarray(T[:, ::-1, ::-1]))
    assert np.allclose(dw, O.wbmm_forward(x, w, T=T), rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- shifted grid
def brute_force_shifted(x, T, w, oy, ox):
    """Per-output sum over the positions of the output's own window, windows starting at
    k*w - oy (rows) and k*w - ox (columns), pure Python loops."""
    B, C, H, W = x.shape
    out = np.zeros((B, C, H, W))
    for b in range(B):
        for c in range(C):
            for py in range(H):
                for px in range(W):
                    wy0 = ((py + oy) // w) * w - oy
                    wx0 = ((px + ox) // w) * w - ox
                    acc = 0.0
                    for qy in range(max(wy0, 0), min(wy0 + w, H)):
                        for qx in range(max(wx0, 0), min(wx0 + w, W)):
                            acc += T[c, py - qy + w - 1, px - qx + w - 1] * x[b, c, qy, qx]
                    out[b, c, py, px] = acc
    return out


@pytest.mark.parametrize("B,C,H,W,w,oy,ox", [(1, 2, 9, 11, 4, 2, 2), (2, 1, 7, 7, 7, 3, 3),
                                              (1, 2, 10, 6, 3, 1, 2), (1, 1, 5, 9, 5, 0, 4)])
def test_shifted_brute_force(B, C, H, W, w, oy, ox):
    x = rnd((B, C, H, W), seed=300 + w)
    T = rnd((C, 2 * w - 1, 2 * w - 1), 0.1, seed=301 + w)
    assert np.allclose(O.wbmm_forward_shifted(x, w, oy, ox, T=T),
                       brute_force_shifted(x, T, w, oy, ox), rtol=0, atol=1e-12)


def test_shifted_zero_offset_is_plain():
    x = rnd((2, 3, 13, 10), seed=310)
    T = rnd((3, 9, 9), 0.1, seed=311)
    assert np.array_equal(O.wbmm_forward_shifted(x, 5, 0, 0, T=T), O.wbmm_forward(x, 5, T=T))


def test_shifted_window_borders_move():
    """With a one-hot table that copies the left neighbour, a pixel whose left neighbour lies in
    another window gets 0: at columns k*w - ox, not at the plain grid's k*w."""
    w, ox = 4, 2
    x = rnd((1, 1, 4, 12), seed=320)
    T = np.zeros((1, 7, 7))
    T[0, 3, 4] = 1.0      # offset (0, +1): out[px] = x[px - 1] inside the window
    y = O.wbmm_forward_shifted(x, w, 0, ox, T=T)
    for px in range(12):
        starts_window = (px + ox) % w == 0
        want = 0.0 if starts_window or px == 0 else x[0, 0, :, px - 1]  # px 0: neighbour off-map
        assert np.array_equal(y[0, 0, :, px], np.broadcast_to(want, (4,)))


def rolled_masked_layer(x, T, w, oy, ox):
    """The half-window offset grid computed the way the rolled-map kernels do: roll the map by
    (-oy, -ox), take the plain grid's windows, keep only the pairs whose pixels come from one
    piece (quadrants that agree on every axis the roll split: the last window row when oy != 0,
    the last window column when ox != 0), then roll the result back. Written with numpy from
    that description, not from the oracle."""
    B, C, H, W = x.shape
    h = w // 2
    xr = np.roll(x, (-oy, -ox), axis=(2, 3))
    nwy, nwx = H // w, W // w
    py, px = np.divmod(np.arange(w * w), w)
    out = np.zeros_like(xr)
    for wy in range(nwy):
        for wx in range(nwx):
            ry = oy != 0 and wy == nwy - 1
            rx = ox != 0 and wx == nwx - 1
            same = np.ones((w * w, w * w), bool)
            if ry:
                same &= (py[:, None] // h) == (py[None, :] // h)
            if rx:
                same &= (px[:, None] // h) == (px[None, :] // h)
            for c in range(C):
                M = T[c][py[:, None] - py[None, :] + w - 1, px[:, None] - px[None, :] + w - 1]
                Mm = np.where(same, M, 0.0)
                blk = xr[:, c, wy * w:(wy + 1) * w, wx * w:(wx + 1) * w].reshape(B, w * w)
                out[:, c, wy * w:(wy + 1) * w, wx * w:(wx + 1) * w] = \
                    (blk @ Mm.T).reshape(B, w, w)
    return np.roll(out, (oy, ox), axis=(2, 3))


@pytest.mark.parametrize("H,oy,ox", [(28, 7, 7), (28, 7, 0), (28, 0, 7), (56, 7, 7), (14, 7, 7)])
def test_rolled_map_equals_offset_grid(H, oy, ox):
    """The identity the rolled-map kernels rest on: with w = 14 and offsets of 0 or w / 2 on maps
    whose sides are multiples of w, the layer on the offset grid (zero-padded border windows) is
    the masked plain-grid product on the rolled map, rolled back."""
    w = 14
    x = rnd((2, 2, H, H), seed=340 + H)
    T = rnd((2, 2 * w - 1, 2 * w - 1), 0.1, seed=341)
    assert np.allclose(O.wbmm_forward_shifted(x, w, oy, ox, T=T),
                       rolled_masked_layer(x, T, w, oy, ox), rtol=0, atol=1e-12)


def test_rolled_map_without_mask_differs():
    """Without the mask the rolled map's plain product mixes pixels of different offset windows:
    the identity above depends on the mask (a check that the pin can fail)."""
    w, H = 14, 28
    x = rnd((1, 1, H, H), seed=350)
    T = rnd((1, 27, 27), 0.1, seed=351)
    plain_rolled = np.roll(O.wbmm_forward(np.roll(x, (-7, -7), axis=(2, 3)), w, T=T), (7, 7),
                           axis=(2, 3))
    assert not np.allclose(O.wbmm_forward_shifted(x, w, 7, 7, T=T), plain_rolled, atol=1e-6)


@pytest.mark.parametrize("oy,ox", [(2, 3), (3, 0)])
def test_shifted_backward_adjoint_and_fd(oy, ox):
    """dx by the adjoint identity <WBMM_s(x), g> = <x, dX_s(g)>; dT by central differences of
    L(T) = sum(g * WBMM_s(x; T)) (linear in T, so exact up to rounding)."""
    w = 5
    x = rnd((2, 2, 11, 8), seed=330)
    g = rnd((2, 2, 11, 8), seed=331)
    T = rnd((2, 9, 9), 0.1, seed=332)
    dx, dT = O.wbmm_backward_shifted(x, g, w, oy, ox, T=T)
    y = O.wbmm_forward_shifted(x, w, oy, ox, T=T)
    assert abs(np.sum(y * g) - np.sum(dx * x)) < 1e-9
    eps = 1e-3
    for c, i, j in [(0, 4, 4), (1, 0, 8), (0, 7, 2), (1, 3, 6)]:
        Tp, Tm = T.copy(), T.copy()
        Tp[c, i, j] += eps
        Tm[c, i, j] -= eps
        fd = (np.sum(g * O.wbmm_forward_shifted(x, w, oy, ox, T=Tp)) -
              np.sum(g * O.wbmm_forward_shifted(x, w, oy, ox, T=Tm))) / (2 * eps)
        assert abs(fd - dT[c, i, j]) < 1e-8 * max(1.0, abs(fd))


def mix_brute_force(z, Wm):
    """3x3 depthwise cross-correlation with zero padding 1, pure Python loops."""
    B, C, H, W = z.shape
    out = np.zeros_like(z, dtype=np.float64)
    for b in range(B):
        for c in range(C):
            for py in range(H):
                for px in range(W):
                    acc = 0.0
                    for u in range(3):
                        for t in range(3):
                            qy, qx = py + u - 1, px + t - 1
                            if 0 <= qy < H and 0 <= qx < W:
                                acc += Wm[c, u, t] * z[b, c, qy, qx]
                    out[b, c, py, px] = acc
    return out


@pytest.mark.parametrize("B,C,H,W,w,oy,ox", [(1, 2, 9, 11, 4, 2, 2), (2, 1, 10, 7, 5, 4, 1)])
def test_shifted_layer_with_mix_brute_force(B, C, H, W, w, oy, ox):
    """The interleaved layer is the offset-grid WBMM followed by the 3x3 mix on the map itself
    (zero padding at the map border, not at the padded grid's): both stages as pure loops."""
    x = rnd((B, C, H, W), seed=340 + w)
    T = rnd((C, 2 * w - 1, 2 * w - 1), 0.1, seed=341 + w)
    Wm = rnd((C, 3, 3), 0.1, seed=342 + w)
    y, z = O.layer_forward_shifted(x, w, oy, ox, T=T, Wmix=Wm)
    zb = brute_force_shifted(x, T, w, oy, ox)
    assert np.allclose(z, zb, rtol=0, atol=1e-12)
    assert np.allclose(y, mix_brute_force(zb, Wm), rtol=0, atol=1e-12)
    # the cached-matrix form gives the same layer
    y2, z2 = O.layer_forward_shifted(x, w, oy, ox, M=O.build_matrix(T, w), Wmix=Wm)
    assert np.array_equal(y2, y) and np.array_equal(z2, z)


@pytest.mark.parametrize("oy,ox", [(2, 3), (4, 0)])
def test_shifted_layer_with_mix_finite_differences(oy, ox):
    """Central differences of L = sum(dY * y) through the offset grid and the mix, for entries of
    x, T and the mix weights: L is linear in each, so the differences are exact up to rounding.
    A mix applied on the padded grid, or dY used in place of the mix adjoint, fails this."""
    w = 5
    x = rnd((2, 2, 11, 8), seed=350)
    T = rnd((2, 9, 9), 0.1, seed=351)
    Wm = rnd((2, 3, 3), 0.2, seed=352)
    dY = rnd((2, 2, 11, 8), seed=353)
    dx, dT, dW = O.layer_backward_shifted(x, dY, w, oy, ox, T=T, Wmix=Wm)
    # z passed in (as the GPU backward gets it) or recomputed: the same gradients
    _, z = O.layer_forward_shifted(x, w, oy, ox, T=T, Wmix=Wm)
    dx2, dT2, dW2 = O.layer_backward_shifted(x, dY, w, oy, ox, T=T, Wmix=Wm, z=z)
    assert np.array_equal(dx, dx2) and np.array_equal(dT, dT2) and np.array_equal(dW, dW2)
    dx3, dT3, dW3 = O.layer_backward_shifted(x, dY, w, oy, ox, M=O.build_matrix(T, w), Wmix=Wm,
                                             z=z)
    assert np.allclose(dx3, dx, rtol=0, atol=1e-12) and np.allclose(dT3, dT, rtol=0, atol=1e-12)

    def L(x_=x, T_=T, W_=Wm):
        return np.sum(dY * brute_force_layer_shifted(x_, T_, W_, w, oy, ox))

    h = 1e-3

    def fd(arr, k, key):
        P, Mn = arr.copy().reshape(-1), arr.copy().reshape(-1)
        P[k] += h
        Mn[k] -= h
        return (L(**{key: P.reshape(arr.shape)}) - L(**{key: Mn.reshape(arr.shape)})) / (2 * h)

    for k in (0, 17, 40, 80, 161):
        assert abs(fd(T, k, "T_") - dT.reshape(-1)[k]) <= 1e-8
    for k in range(Wm.size):
        assert abs(fd(Wm, k, "W_") - dW.reshape(-1)[k]) <= 1e-8
    for k in (0, 9, 50, 87, 200, 351):
        assert abs(fd(x, k, "x_") - dx.reshape(-1)[k]) <= 1e-8


def brute_force_layer_shifted(x, T, Wm, w, oy, ox):
    return mix_brute_force(brute_force_shifted(x, T, w, oy, ox), Wm)
