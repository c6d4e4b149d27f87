"""WBMM oracle: a plain, slow, obviously-correct CPU implementation in float64.

TEST INFRASTRUCTURE ONLY. Only the test suite, ``__graft_entry__.smoke()`` and the bench's
``cpu_baseline`` leg may import this module. The library under ``receptive_field_spatial_amd``
never imports it and has no CPU fallback; nothing here is shared with the HIP path.

What it computes (WBMM, "Windowed Batch Matrix Multiplication"):
  * the feature map is cut into non-overlapping w x w windows (d = w*w pixels each)
    [gecl.asia reading notes, "Core Idea"; arxivdaily abstract];
  * a compact per-channel table T_c of (2w-1) x (2w-1) relative-offset weights is indexed by the
    offset between two in-window positions to give a d x d matrix M_c
    [gecl.asia reading notes, "Core Idea" and "Method" point 2];
  * every window of every image is mixed by one shared matmul out = M_c . x, with no softmax and
    no input dependence in the weights [gecl.asia reading notes, "Relation To Prior Work"];
  * windows do not talk to each other; an optional 3x3 depthwise mix afterwards restores
    cross-window flow, an optional 7x7 sub-table is folded into a 14x14 window's matrix, and M
    may be cached for inference [gecl.asia reading notes, "Method" points 3-4 and last sentence].

Readings taken where the pages leave a step open:
  R1 offset orientation: M[i,j] = T[(y_i - y_j) + w - 1, (x_i - x_j) + w - 1], first table axis
     vertical; R2 in-window order i = y*w + x, windows ordered (b, wy, wx) row-major;
  R3 H, W not multiples of w are zero-padded at the bottom/right and the output is cropped;
  R4 the 3x3 mix is a depthwise cross-correlation (zero pad 1, stride 1, no bias) applied after
     the window mixer on the cropped map;
  R5 the hierarchical fold is additive on same-sub-window pairs (s | w), one float32 RNE add;
  R9 gradients are returned, not accumulated.

Every function works in float64 on the exact values the GPU receives (float32 values, or bf16
values widened), except ``fold_hier`` which reproduces the single float32 addition bit-exactly.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

__all__ = [
    "padded_hw", "build_index", "build_matrix", "fold_hier", "sub_index",
    "pad_map", "partition", "reverse", "wbmm_forward", "mix_forward", "mix_backward",
    "wbmm_backward", "layer_forward", "layer_backward", "wbmm_backward_hier",
    "layer_forward_hier", "layer_backward_hier", "dw_conv_forward",
    "wbmm_forward_shifted", "wbmm_backward_shifted", "layer_forward_shifted",
    "layer_backward_shifted",
]


# ----------------------------------------------------------------------------- geometry
def padded_hw(H: int, W: int, w: int) -> Tuple[int, int]:
    """Padded map size: the next multiples of w (reading R3)."""
    return -(-H // w) * w, -(-W // w) * w


def _coords(w: int) -> Tuple[np.ndarray, np.ndarray]:
    i = np.arange(w * w)
    return i // w, i % w


def build_index(w: int) -> np.ndarray:
    """Relative-position index idx[i, j] (int32, d x d).

    The pages describe indexing a compact relative-position table by the offset between the two
    in-window positions [gecl.asia reading notes, "Core Idea"]; with reading R1 the flat table
    index of the offset (dy, dx) = (y_i - y_j, x_i - x_j) is (dy + w - 1) * (2w - 1) + (dx + w - 1).
    """
    y, x = _coords(w)
    dy = y[:, None] - y[None, :]
    dx = x[:, None] - x[None, :]
    return ((dy + w - 1) * (2 * w - 1) + (dx + w - 1)).astype(np.int32)


def build_matrix(T: np.ndarray, w: int) -> np.ndarray:
    """M[c, i, j] = T[c].flat[idx[i, j]] — an exact gather, dtype preserved.

    Per-channel d x d weight matrix built by indexing the table
    [gecl.asia reading notes, "Core Idea"; arxivdaily abstract].
    """
    C = T.shape[0]
    assert T.shape[1:] == (2 * w - 1, 2 * w - 1)
    return T.reshape(C, -1)[:, build_index(w)]


def sub_index(w: int, s: int) -> Tuple[np.ndarray, np.ndarray]:
    """For the hierarchical fold: (same-sub-window mask, sub-table index) over d x d pairs.

    Reading R5: sub-windows are the s x s blocks of the w x w window aligned to its origin; a pair
    (i, j) is inside one sub-window when (y//s, x//s) agree; its sub-table index uses the same
    convention as build_index with s in place of w.
    """
    y, x = _coords(w)
    same = ((y[:, None] // s) == (y[None, :] // s)) & ((x[:, None] // s) == (x[None, :] // s))
    ys, xs = y % s, x % s
    idx_s = (ys[:, None] - ys[None, :] + s - 1) * (2 * s - 1) + (xs[:, None] - xs[None, :] + s - 1)
    return same, idx_s.astype(np.int32)


def fold_hier(M: np.ndarray, T_sub: np.ndarray, w: int, s: int) -> np.ndarray:
    """Fold an s x s sub-window table into the w x w matrix (hierarchical reparameterization).

    The pages overlay 7x7 local structure inside a 14x14 window at no inference cost
    [gecl.asia reading notes, "Method" point 4]. Reading R5: additive, one add in M's own dtype
    (numpy float32 addition is IEEE round-to-nearest-even), only for same-sub-window pairs.
    """
    assert w % s == 0 and 1 <= s < w
    same, idx_s = sub_index(w, s)
    C = M.shape[0]
    add = T_sub.reshape(C, -1)[:, idx_s].astype(M.dtype)
    out = M.copy()
    out[:, same] = (M[:, same] + add[:, same]).astype(M.dtype)
    return out


# ----------------------------------------------------------------------------- partition
def pad_map(x: np.ndarray, w: int) -> np.ndarray:
    """Zero-pad (B, C, H, W) at the bottom/right to multiples of w (reading R3)."""
    B, C, H, W = x.shape
    Hp, Wp = padded_hw(H, W, w)
    out = np.zeros((B, C, Hp, Wp), dtype=np.float64)
    out[:, :, :H, :W] = x
    return out


def partition(xp: np.ndarray, w: int) -> np.ndarray:
    """Padded map (B, C, Hp, Wp) -> window-major X (C, d, N), N = B * nH * nW.

    X[c, y*w + x, (b*nH + wy)*nW + wx] = xp[b, c, wy*w + y, wx*w + x]
    [gecl.asia reading notes, "Core Idea": the input is cut into contiguous windows].
    """
    B, C, Hp, Wp = xp.shape
    nH, nW = Hp // w, Wp // w
    t = xp.reshape(B, C, nH, w, nW, w).transpose(1, 3, 5, 0, 2, 4)  # (C, y, x, B, nH, nW)
    return t.reshape(C, w * w, B * nH * nW)


def reverse(Z: np.ndarray, B: int, Hp: int, Wp: int, w: int) -> np.ndarray:
    """Inverse of ``partition``: (C, d, N) -> (B, C, Hp, Wp)."""
    C = Z.shape[0]
    nH, nW = Hp // w, Wp // w
    t = Z.reshape(C, w, w, B, nH, nW).transpose(3, 0, 4, 1, 5, 2)  # (B, C, nH, y, nW, x)
    return t.reshape(B, C, Hp, Wp)


# ----------------------------------------------------------------------------- forward
def _matrices(w: int, T: Optional[np.ndarray], M: Optional[np.ndarray]) -> np.ndarray:
    if (T is None) == (M is None):
        raise ValueError("exactly one of T (table) or M (cached matrix) must be given")
    return build_matrix(T, w) if M is None else M


def wbmm_forward(x: np.ndarray, w: int, T: Optional[np.ndarray] = None,
                 M: Optional[np.ndarray] = None) -> np.ndarray:
    """WBMM output (B, C, H, W) in float64.

    Steps in the pages' order [gecl.asia reading notes, "Core Idea"; pith page, "Core claim"]:
    pad + partition into windows, index the table into M_c, one matmul per channel shared by all
    windows of all images (no softmax), then put the windows back and crop.
    """
    B, C, H, W = x.shape
    Hp, Wp = padded_hw(H, W, w)
    Mc = _matrices(w, T, M)
    X = partition(pad_map(x, w), w)
    Z = np.empty_like(X)
    for c in range(C):
        Z[c] = Mc[c].astype(np.float64) @ X[c]
    return reverse(Z, B, Hp, Wp, w)[:, :, :H, :W]


def mix_forward(z: np.ndarray, Wmix: np.ndarray) -> np.ndarray:
    """3x3 depthwise inter-block mix (reading R4): y[b,c,h,v] = sum_{u,t} W[c,u,t] z_pad[b,c,h+u,v+t].

    The pages add cross-block 3x3 depthwise mixing to connect neighbouring windows
    [gecl.asia reading notes, "Method" point 3]; z_pad is z with one zero pixel on each side.
    """
    B, C, H, W = z.shape
    zp = np.zeros((B, C, H + 2, W + 2), dtype=np.float64)
    zp[:, :, 1:-1, 1:-1] = z
    Wd = Wmix.astype(np.float64)
    y = np.zeros((B, C, H, W), dtype=np.float64)
    for u in range(3):
        for t in range(3):
            y += Wd[None, :, u, t, None, None] * zp[:, :, u:u + H, t:t + W]
    return y


def dw_conv_forward(x: np.ndarray, Wdw: np.ndarray) -> np.ndarray:
    """Standard k x k depthwise convolution (the pages' DW-Std baseline, reading R18).

    Every output gathers the k*k neighbours around its own position from its own channel
    [pith page, Fig. 1 and Fig. 2 captions]; it is the operator the pages time WBMM against
    [pith page, Fig. 3 caption]. Written as the deep-learning frameworks define it:
    y[b,c,h,v] = sum_{u,t} W[c,u,t] * x_pad[b,c,h+u,v+t], x_pad = x with p = k // 2 zero pixels
    on every side, odd k, stride 1, no bias.
    """
    B, C, H, W = x.shape
    k = Wdw.shape[-1]
    assert Wdw.shape == (C, k, k) and k % 2 == 1
    p = k // 2
    xp = np.zeros((B, C, H + 2 * p, W + 2 * p), dtype=np.float64)
    xp[:, :, p:p + H, p:p + W] = x
    Wd = Wdw.astype(np.float64)
    y = np.zeros((B, C, H, W), dtype=np.float64)
    for u in range(k):
        for t in range(k):
            y += Wd[None, :, u, t, None, None] * xp[:, :, u:u + H, t:t + W]
    return y


def mix_backward(dy: np.ndarray, z: np.ndarray, Wmix: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Gradients of ``mix_forward``: (dz, dWmix), derived by the chain rule (reading R9)."""
    B, C, H, W = dy.shape
    dyp = np.zeros((B, C, H + 2, W + 2), dtype=np.float64)
    dyp[:, :, 1:-1, 1:-1] = dy
    zp = np.zeros_like(dyp)
    zp[:, :, 1:-1, 1:-1] = z
    Wd = Wmix.astype(np.float64)
    dz = np.zeros((B, C, H, W), dtype=np.float64)
    dW = np.zeros((C, 3, 3), dtype=np.float64)
    for u in range(3):
        for t in range(3):
            # z[h, v] feeds y[h - u + 1, v - t + 1] with weight W[u, t].
            dz += Wd[None, :, u, t, None, None] * dyp[:, :, 2 - u:2 - u + H, 2 - t:2 - t + W]
            dW[:, u, t] = np.einsum("bchv,bchv->c", dy.astype(np.float64),
                                    zp[:, :, u:u + H, t:t + W])
    return dz, dW


def wbmm_backward(x: np.ndarray, dz: np.ndarray, w: int, T: Optional[np.ndarray] = None,
                  M: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Gradients of ``wbmm_forward`` given dL/dz: (dx, dT), float64.

    The pages report training with the operator but do not spell out its backward; it follows by
    calculus from the forward: dX_c = M_c^T G_c and dM_c = G_c X_c^T, and since M_c only copies
    table entries, dT_c[k] is the sum of dM_c over the pairs whose index is k.
    """
    B, C, H, W = x.shape
    Hp, Wp = padded_hw(H, W, w)
    Mc = _matrices(w, T, M)
    X = partition(pad_map(x, w), w)
    G = partition(pad_map(dz, w), w)
    idx = build_index(w).ravel()
    L = (2 * w - 1) ** 2
    dX = np.empty_like(X)
    dT = np.empty((C, L), dtype=np.float64)
    for c in range(C):
        dX[c] = Mc[c].astype(np.float64).T @ G[c]
        P = G[c] @ X[c].T
        dT[c] = np.bincount(idx, weights=P.ravel(), minlength=L)
    dx = reverse(dX, B, Hp, Wp, w)[:, :, :H, :W]
    return dx, dT.reshape(C, 2 * w - 1, 2 * w - 1)


def wbmm_backward_hier(x: np.ndarray, dz: np.ndarray, w: int, s: int, T: np.ndarray,
                       T_sub: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients of the hierarchical forward, z = M' . x with M' = fold_hier(M(T), T_sub):
    (dx, dT, dT_sub), float64.

    The pages overlay an s x s sub-window table on the w x w window [gecl.asia reading notes,
    "Method" point 4] and train the result, but do not write its backward. By the chain rule, with
    dM_c = G_c X_c^T per channel: dX_c = M'_c^T G_c; M' copies T_c[idx] at every pair, so dT_c[k]
    is the sum of dM_c over the pairs with idx = k (as without the fold); M' adds T_sub_c[idx_s]
    only at same-sub-window pairs (reading R5), so dT_sub_c[k'] is the sum of dM_c over the
    same-sub-window pairs with idx_s = k'. M' is formed in T's dtype (float32 tables give the
    float32-rounded fold).
    """
    B, C, H, W = x.shape
    Hp, Wp = padded_hw(H, W, w)
    Mf = fold_hier(build_matrix(T, w), T_sub, w, s)
    X = partition(pad_map(x, w), w)
    G = partition(pad_map(dz, w), w)
    idx = build_index(w).ravel()
    same, idx_s = sub_index(w, s)
    L, Ls = (2 * w - 1) ** 2, (2 * s - 1) ** 2
    dX = np.empty_like(X)
    dT = np.empty((C, L), dtype=np.float64)
    dTs = np.empty((C, Ls), dtype=np.float64)
    for c in range(C):
        dX[c] = Mf[c].astype(np.float64).T @ G[c]
        P = G[c] @ X[c].T
        dT[c] = np.bincount(idx, weights=P.ravel(), minlength=L)
        dTs[c] = np.bincount(idx_s[same], weights=P[same], minlength=Ls)
    dx = reverse(dX, B, Hp, Wp, w)[:, :, :H, :W]
    return dx, dT.reshape(C, 2 * w - 1, 2 * w - 1), dTs.reshape(C, 2 * s - 1, 2 * s - 1)


# ----------------------------------------------------------------------------- full layer
def layer_forward(x, w, T=None, M=None, Wmix=None):
    """WBMM then, if Wmix is given, the 3x3 mix. Returns (y, z) with z the pre-mix output."""
    z = wbmm_forward(x, w, T=T, M=M)
    y = mix_forward(z, Wmix) if Wmix is not None else z
    return y, z


def layer_backward(x, dy, w, T=None, M=None, Wmix=None, z=None):
    """Backward of ``layer_forward``: (dx, dT, dWmix-or-None)."""
    if Wmix is not None:
        if z is None:
            z = wbmm_forward(x, w, T=T, M=M)
        dz, dW = mix_backward(dy, z, Wmix)
    else:
        dz, dW = dy.astype(np.float64), None
    dx, dT = wbmm_backward(x, dz, w, T=T, M=M)
    return dx, dT, dW


# ----------------------------------------------------------------------------- shifted grid
def _shift_pad(x: np.ndarray, oy: int, ox: int) -> np.ndarray:
    B, C, H, W = x.shape
    out = np.zeros((B, C, H + oy, W + ox), dtype=np.float64)
    out[:, :, oy:, ox:] = x
    return out


def wbmm_forward_shifted(x: np.ndarray, w: int, oy: int, ox: int, T=None, M=None) -> np.ndarray:
    """WBMM on a window grid offset by (oy, ox), 0 <= oy, ox < w (reading R19).

    The pages list interleaving the window grid between layers as a way to let information cross
    window borders, without defining it [gecl.asia reading notes, "Limitations"]. Taken: the
    windows of such a layer cover map rows [k w - oy, (k+1) w - oy) and columns likewise; pixels
    of a border window that fall outside the map are zeros (as for ragged maps, reading R3).
    Written as: oy zero rows on top and ox zero columns on the left, the plain forward, then the
    added rows and columns removed.
    """
    H, W = x.shape[2:]
    return wbmm_forward(_shift_pad(x, oy, ox), w, T=T, M=M)[:, :, oy:oy + H, ox:ox + W]


def wbmm_backward_shifted(x, dz, w, oy, ox, T=None, M=None):
    """Gradients of ``wbmm_forward_shifted``: (dx, dT). The padding pixels are constants, so dx is
    the padded problem's dx without them and dT is the padded problem's dT (zeros add nothing)."""
    H, W = x.shape[2:]
    dx, dT = wbmm_backward(_shift_pad(x, oy, ox), _shift_pad(dz, oy, ox), w, T=T, M=M)
    return dx[:, :, oy:oy + H, ox:ox + W], dT


def layer_forward_shifted(x, w, oy, ox, T=None, M=None, Wmix=None):
    """Shifted-grid WBMM, then the optional 3x3 mix on the map. Returns (y, z)."""
    z = wbmm_forward_shifted(x, w, oy, ox, T=T, M=M)
    y = mix_forward(z, Wmix) if Wmix is not None else z
    return y, z


def layer_backward_shifted(x, dy, w, oy, ox, T=None, M=None, Wmix=None, z=None):
    """Backward of ``layer_forward_shifted``: (dx, dT, dWmix-or-None)."""
    if Wmix is not None:
        if z is None:
            z = wbmm_forward_shifted(x, w, oy, ox, T=T, M=M)
        dz, dW = mix_backward(dy, z, Wmix)
    else:
        dz, dW = dy.astype(np.float64), None
    dx, dT = wbmm_backward_shifted(x, dz, w, oy, ox, T=T, M=M)
    return dx, dT, dW


def layer_forward_hier(x, w, s, T, T_sub, Wmix=None):
    """Hierarchical layer: WBMM with M' = fold_hier(M(T), T_sub), then the optional 3x3 mix.
    Returns (y, z)."""
    z = wbmm_forward(x, w, M=fold_hier(build_matrix(T, w), T_sub, w, s))
    y = mix_forward(z, Wmix) if Wmix is not None else z
    return y, z


def layer_backward_hier(x, dy, w, s, T, T_sub, Wmix=None, z=None):
    """Backward of ``layer_forward_hier``: (dx, dT, dT_sub, dWmix-or-None)."""
    if Wmix is not None:
        if z is None:
            _, z = layer_forward_hier(x, w, s, T, T_sub)
        dz, dW = mix_backward(dy, z, Wmix)
    else:
        dz, dW = dy.astype(np.float64), None
    dx, dT, dTs = wbmm_backward_hier(x, dz, w, s, T, T_sub)
    return dx, dT, dTs, dW
