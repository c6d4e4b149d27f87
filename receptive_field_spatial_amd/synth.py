"""Seeded synthetic inputs for the WBMM workloads.

This module only draws random tensors and names workload shapes; it contains none of the
operator's arithmetic. It is the one piece shared by the oracle-side tests, the GPU parity
tests, ``smoke()`` and the bench, so both sides of every comparison see identical inputs.

Recipe (applied to every workload):
  * generator: ``numpy.random.default_rng(seed)`` (PCG64), seed 0 unless a test says otherwise;
  * draw order: x, T, T_sub, Wmix, dY (only the tensors a workload uses are drawn);
  * each tensor is ``standard_normal`` in float64 times sigma (sigma is a standard deviation),
    then cast to float32 (round-to-nearest-even);
  * bf16 workloads round the float32 values once more to bfloat16 (round-to-nearest-even on the
    bit pattern); both the GPU and the oracle then consume those same bf16 values.

The shapes stand in for the pages' workloads (ImageNet-stage feature maps, a high-resolution
dense-prediction map, a training-shaped later stage); no dataset or trained weight is used.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np


# ----------------------------------------------------------------------------- bf16 helpers
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even) and return the uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 value, returned as float32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(a))


# ----------------------------------------------------------------------------- workloads
@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    C: int
    H: int
    W: int
    w: int
    dtype: str = "f32"           # "f32" or "bf16" (input precision; accumulation is fp32)
    sigma_T: float = 0.02
    s: Optional[int] = None       # hierarchical sub-window size (fold), None = no fold
    sigma_Tsub: float = 0.02
    mix: bool = False             # 3x3 depthwise inter-block mix after the window mixer
    sigma_mix: float = 0.1
    backward: bool = False        # draw dY and run the backward pass
    shift: int = 0                # window grid offset (shift, shift) of an interleaved layer
    note: str = ""

    @property
    def d(self) -> int:
        return self.w * self.w


WORKLOADS: Dict[str, Workload] = {
    "tiny_w7": Workload("tiny_w7", B=1, C=8, H=28, W=28, w=7,
                        note="tiny fp32 forward, 16 windows"),
    "stage1_w14": Workload("stage1_w14", B=128, C=96, H=56, W=56, w=14,
                           note="fp32 forward at an ImageNet stage-1 shape"),
    "bf16_w7": Workload("bf16_w7", B=64, C=192, H=56, W=56, w=7, dtype="bf16",
                        note="bf16 window sweep"),
    "bf16_w14": Workload("bf16_w14", B=64, C=192, H=56, W=56, w=14, dtype="bf16",
                         note="bf16 window sweep"),
    "bf16_w28": Workload("bf16_w28", B=64, C=192, H=56, W=56, w=28, dtype="bf16",
                         note="bf16 window sweep"),
    "highres_w14": Workload("highres_w14", B=2, C=128, H=128, W=128, w=14, s=7, mix=True,
                            note="dense-prediction map padded 128->140, fold + 3x3 mix"),
    "train_w14": Workload("train_w14", B=64, C=192, H=28, W=28, w=14, mix=True, backward=True,
                          note="fp32 training step: forward + backward with 3x3 mix"),
    "train_w14_bf16": Workload("train_w14_bf16", B=64, C=192, H=28, W=28, w=14, dtype="bf16",
                               backward=True,
                               note="bf16 (mixed-precision) training step of the operator"),
    "train_w14_bf16_mix": Workload("train_w14_bf16_mix", B=64, C=192, H=28, W=28, w=14,
                                   dtype="bf16", mix=True, backward=True,
                                   note="bf16 training step of the layer with the 3x3 mix"),
    "train_w14_shift": Workload("train_w14_shift", B=64, C=192, H=28, W=28, w=14, mix=True,
                                backward=True, shift=7,
                                note="fp32 training step of an interleaved layer (grid offset 7)"),
    "train_stage1_shift": Workload("train_stage1_shift", B=32, C=96, H=56, W=56, w=14, mix=True,
                                   backward=True, shift=7,
                                   note="fp32 training step of an interleaved layer at the stage-1 "
                                        "map size (grid offset 7)"),
    "train_w14_hier": Workload("train_w14_hier", B=64, C=192, H=28, W=28, w=14, s=7, mix=True,
                               backward=True,
                               note="fp32 training step with the 7x7 sub-window table folded on "
                                    "chip and its gradient"),
}


def draw_inputs(wl: Workload, seed: int = 0, *, B: Optional[int] = None,
                C: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw the workload's tensors (float32; bf16 workloads get bf16-valued float32 for x/T).

    ``B``/``C`` override the batch or channel count (used for reduced parity cases); the draw
    order and recipe stay the same.
    """
    B = wl.B if B is None else B
    C = wl.C if C is None else C
    rng = np.random.default_rng(seed)

    def normal(shape, sigma):
        return (rng.standard_normal(shape, dtype=np.float64) * sigma).astype(np.float32)

    L = 2 * wl.w - 1
    out: Dict[str, np.ndarray] = {}
    out["x"] = normal((B, C, wl.H, wl.W), 1.0)
    out["T"] = normal((C, L, L), wl.sigma_T)
    if wl.s is not None:
        Ls = 2 * wl.s - 1
        out["T_sub"] = normal((C, Ls, Ls), wl.sigma_Tsub)
    if wl.mix:
        out["Wmix"] = normal((C, 3, 3), wl.sigma_mix)
    if wl.backward:
        out["dY"] = normal((B, C, wl.H, wl.W), 1.0)
    if wl.dtype == "bf16":
        out["x"] = round_to_bf16(out["x"])
        out["T"] = round_to_bf16(out["T"])
        if wl.backward:
            out["dY"] = round_to_bf16(out["dY"])
    return out


def normal_f32(shape, sigma: float = 1.0, seed: int = 0) -> np.ndarray:
    """One seeded N(0, sigma) float32 tensor (helper for ad-hoc test shapes)."""
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(shape, dtype=np.float64) * sigma).astype(np.float32)
