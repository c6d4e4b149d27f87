"""The allocation-free backward (wbmm_backward_noalloc) against wbmm_backward with a caller
workspace, through the C ABI: two calls in a row on the same GPU scratch, the second with a
smaller input, each compared with the workspace call (same kernels: bit for bit) and with the
oracle. Outputs are preallocated, so the calls allocate nothing."""
import numpy as np
import pytest

from oracle import wbmm_oracle as O
from receptive_field_spatial_amd import synth
from tests.parity_util import assert_f32

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def R():
    import receptive_field_spatial_amd as mod
    mod.load_library()
    return mod


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def one_call(B, C, H, W, w, mix, seed, cached=False):
    print(f"\n[case] noalloc B={B} C={C} H={H} W={W} w={w} mix={mix} cached={cached}", flush=True)
    x = synth.normal_f32((B, C, H, W), 1.0, seed=seed)
    T = synth.normal_f32((C, 2 * w - 1, 2 * w - 1), 0.02, seed=seed + 1)
    Wm = synth.normal_f32((C, 3, 3), 0.1, seed=seed + 2) if mix else None
    dy = synth.normal_f32((B, C, H, W), 1.0, seed=seed + 3)
    xd, Td, dyd = dev(x), dev(T), dev(dy)
    kw = {"M": R().wbmm_build_matrix(Td, w)} if cached else {"T": Td}
    Wd = dev(Wm) if mix else None
    zs = None
    if mix:
        zs = torch.empty_like(xd)
        R().wbmm_forward(xd, w, mix_w=Wd, z_save=zs, **kw)
    L = 2 * w - 1
    dx = torch.empty_like(xd)
    dT = torch.empty((C, L, L), device="cuda")
    dW = torch.empty((C, 3, 3), device="cuda") if mix else False
    R().wbmm_backward_noalloc(xd, dyd, w, mix_w=Wd, z_saved=zs, dx=dx, dT=dT, dmix_w=dW, **kw)
    rx, rT, rW = R().wbmm_backward(xd, dyd, w, mix_w=Wd, z_saved=zs, **kw)
    torch.cuda.synchronize()
    assert torch.equal(dx, rx) and torch.equal(dT, rT)
    if mix:
        assert torch.equal(dW, rW)
    wdx, wdT, wdW = O.layer_backward(x.astype(np.float64), dy.astype(np.float64), w, T=T, Wmix=Wm,
                                     z=zs.cpu().numpy().astype(np.float64) if mix else None)
    assert_f32(dx.cpu().numpy(), wdx, "dx")
    assert_f32(dT.cpu().numpy(), wdT, "dT")
    if mix:
        assert_f32(dW.cpu().numpy(), wdW, "dWmix")


@pytest.mark.parametrize("big,small", [
    ((32, 24, 28, 28, 14, True), (5, 3, 28, 28, 14, True)),      # fast kernels, part-empty unit
    ((4, 6, 56, 56, 14, True), (2, 2, 14, 14, 14, False)),       # 56x56 then 14x14 fast kernels
    ((2, 3, 100, 100, 14, True), (1, 2, 30, 25, 14, True)),      # general kernels, dz in scratch
    ((3, 4, 17, 23, 5, False), (1, 2, 9, 9, 3, True)),
])
def test_noalloc_matches_workspace_call_twice(big, small):
    one_call(*big, seed=500)
    one_call(*small, seed=510)


def test_noalloc_cached_matrix():
    one_call(3, 4, 28, 28, 14, True, seed=520, cached=True)


def test_noalloc_rejects_problems_beyond_its_scratch():
    Rm = R()
    B, C, H, W, w = 64, 192, 112, 112, 14  # a backward needing more than the fixed scratch
    need = Rm.wbmm_backward_workspace_bytes(B, C, H, W, w, has_mix=True)
    assert need > Rm.WBMM_NOALLOC_SCRATCH_BYTES
    x = torch.empty((1,), device="cuda")
    lib = Rm._lib()
    p = x.data_ptr()
    st = lib.wbmm_backward_noalloc(B, C, H, W, w, 0, p, p + 1024, None, p + 2048, p + 4096,
                                   p + 8192, None, None, None, None)
    assert st == Rm.WBMM_E_UNSUPPORTED
    assert "scratch" in lib.wbmm_last_error().decode()
