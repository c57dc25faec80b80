"""Seeded synthetic inputs for the forward-convolution layers.

This module is shared by the tests, the bench and the smoke check.  It holds
the layer shapes of the five workloads and the recipe that draws their values;
it holds none of the convolution's arithmetic (no output-size formula, no
products, no sums).  Output shapes are computed by whoever consumes a layer:
the oracle with its own formula, the library with its own.

Value recipe (every layer): ``numpy.random.default_rng(seed)`` (PCG64), float64
draws in the order listed in ``_draw``; ``U[a,b]`` is ``rng.uniform(a, b)`` and
``N(0,1)`` is ``rng.standard_normal``.  Values are scaled in float64 and then
rounded once to the storage dtype with round-to-nearest-even:
  * f32:  float64 -> float32 (numpy cast, RNE)
  * f16:  float64 -> float16 (numpy cast, RNE)
  * bf16: float64 -> float32 (RNE) -> bf16 (RNE on the float32 bits)
Both sides of every comparison read exactly these quantised values.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Tuple

import numpy as np

DTYPES = ("f32", "f16", "bf16")
DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}
DTYPE_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
ACT_CODE = {"none": 0, "relu": 1}


@dataclasses.dataclass(frozen=True)
class Layer:
    """One convolution layer: NC(T)HW input, OI(T)HW weight, per-channel bias.

    2-D layers have ``T == KT == 1``, ``pad[0] == 0`` and ``stride[0] == 1``
    and are run through the 2-D entry point.
    """
    name: str
    dtype: str
    N: int
    C_in: int
    T: int
    H: int
    W: int
    C_out: int
    KT: int
    KH: int
    KW: int
    pad: Tuple[int, int, int]      # (t, h, w)
    stride: Tuple[int, int, int]   # (t, h, w)
    act: str
    dims: int                      # 2 or 3
    x_dist: str                    # "U01", "U11", "N01"
    w_dist: str                    # "U11" or "N01", scaled by 1/sqrt(fan_in)
    b_dist: Optional[str]          # "U0.1", "U0.05", "zero"
    # time padding after the last frame when it differs from pad[0] (the
    # causal 3-D convolution pads only before the first frame); None: pad[0]
    pad_t_back: Optional[int] = None
    # 2x2 stride-2 max pooling after the activation, fused into the conv
    pool: bool = False
    # activations channel-packed ([N][C/g][T][H][W][g], g = 16 bytes of
    # channels) instead of plain NC(T)HW
    cpack: bool = False
    # weights packed once at load (libconv_pack_weights) instead of passed
    # as OI(D)HW on every call
    prepacked: bool = False

    @property
    def taps(self) -> int:
        return self.KT * self.KH * self.KW

    @property
    def fan_in(self) -> int:
        return self.C_in * self.taps

    @property
    def x_shape(self) -> Tuple[int, ...]:
        if self.dims == 2:
            return (self.N, self.C_in, self.H, self.W)
        return (self.N, self.C_in, self.T, self.H, self.W)

    @property
    def w_shape(self) -> Tuple[int, ...]:
        if self.dims == 2:
            return (self.C_out, self.C_in, self.KH, self.KW)
        return (self.C_out, self.C_in, self.KT, self.KH, self.KW)

    def with_(self, **kw) -> "Layer":
        return dataclasses.replace(self, **kw)


def _l2(name, dtype, N, C_in, H, W, C_out, k, s, p, act, xd, wd, bd) -> Layer:
    return Layer(name, dtype, N, C_in, 1, H, W, C_out, 1, k, k, (0, p, p),
                 (1, s, s), act, 2, xd, wd, bd)


def _l3(name, dtype, N, C_in, T, H, W, C_out, k, s, p, act, xd, wd, bd) -> Layer:
    return Layer(name, dtype, N, C_in, T, H, W, C_out, k, k, k, (p, p, p),
                 (s, s, s), act, 3, xd, wd, bd)


# The five workloads.  Layers of one workload draw from one generator, in
# list order (x, w, b per layer).  The OCR stack's layers 2-4 are checked and
# benched separately, each on its own U[0,1] input of the shape the previous
# layer produces (non-negative, like the ReLU output that feeds it).
WORKLOADS: Dict[str, Tuple[int, List[Layer]]] = {
    "conv1": (0, [
        _l2("c1", "f32", 1, 3, 32, 32, 8, 3, 1, 1, "none", "U11", "U11", "U0.1"),
    ]),
    "ocr_stack": (1, [
        _l2("c2_L1", "f32", 1, 3, 640, 640, 32, 3, 2, 1, "relu", "U01", "U11", "U0.1"),
        _l2("c2_L2", "f32", 1, 32, 320, 320, 32, 3, 1, 1, "relu", "U01", "U11", "U0.1"),
        _l2("c2_L3", "f32", 1, 32, 320, 320, 64, 1, 1, 0, "relu", "U01", "U11", "U0.1"),
        _l2("c2_L4", "f32", 1, 64, 320, 320, 64, 3, 2, 1, "relu", "U01", "U11", "U0.1"),
    ]),
    "textrec_f16": (2, [
        _l2("c3_A", "f16", 16, 64, 24, 160, 128, 3, 1, 1, "relu", "N01", "N01", "zero"),
        _l2("c3_B", "f16", 16, 128, 12, 80, 256, 1, 1, 0, "none", "N01", "N01", "zero"),
    ]),
    "unet_bf16": (3, [
        _l2("c4_A", "bf16", 2, 640, 64, 64, 640, 3, 1, 1, "none", "N01", "N01", "U0.05"),
        _l2("c4_B", "bf16", 2, 1280, 32, 32, 1280, 3, 1, 1, "none", "N01", "N01", "U0.05"),
    ]),
    "vae3d_f16": (4, [
        _l3("c5_A", "f16", 1, 128, 5, 256, 480, 128, 3, 1, 1, "none", "N01", "N01", "U0.05"),
        _l3("c5_B", "f16", 1, 512, 5, 64, 120, 512, 3, 1, 1, "relu", "N01", "N01", "U0.05"),
    ]),
}

ALL_LAYERS: Dict[str, Layer] = {l.name: l for _, ls in WORKLOADS.values() for l in ls}

# Beyond the five: the OCR conv + pool block, and the video-VAE layers made
# causal in time (KT-1 = 2 frames of padding before the first frame, none
# after), the Convolution3D of the spatio-temporal VAE in "SeedVR2 NCNN
# Vulkan", section 7.2.  Shapes and value distributions of the workloads they
# extend, own seeds.
EXTRA_WORKLOADS: Dict[str, Tuple[int, List[Layer]]] = {
    # the OCR detector's conv + ReLU + 2x2 max-pool block, fused into one call
    # ("PP-OCR on Vulkan compute shaders", section 4.4): the OCR stack's
    # second layer followed by the pooling, 320x320 -> 160x160
    "ocr_pool_f32": (6, [
        _l2("c2p_L2", "f32", 1, 32, 320, 320, 32, 3, 1, 1, "relu", "U01", "U11",
            "U0.1").with_(pool=True),
    ]),
    "vae3d_causal_f16": (5, [
        _l3("c5c_A", "f16", 1, 128, 5, 256, 480, 128, 3, 1, 1, "none", "N01", "N01",
            "U0.05").with_(pad=(2, 1, 1), pad_t_back=0),
        _l3("c5c_B", "f16", 1, 512, 5, 64, 120, 512, 3, 1, 1, "relu", "N01", "N01",
            "U0.05").with_(pad=(2, 1, 1), pad_t_back=0),
    ]),
    # the video-VAE and diffusion-UNet layers on channel-packed activations
    # (the network-wide channel packing of "SeedVR2 NCNN Vulkan", section 9);
    # same shapes and values as the plain-layout workloads
    "vae3d_cpack_f16": (WORKLOADS["vae3d_f16"][0],
                        [l.with_(name=l.name.replace("c5_", "c5x_"), cpack=True)
                         for l in WORKLOADS["vae3d_f16"][1]]),
    # (the OCR stack's weights packed once at load: its plain-layout tiles
    # read OIHW weights, the packed-layout tiles packed ones)
    "ocr_cpack_f32": (WORKLOADS["ocr_stack"][0],
                      [l.with_(name=l.name.replace("c2_", "c2x_"), cpack=True, prepacked=True)
                       for l in WORKLOADS["ocr_stack"][1]]),
    "unet_cpack_bf16": (WORKLOADS["unet_bf16"][0],
                        [l.with_(name=l.name.replace("c4_", "c4x_"), cpack=True)
                         for l in WORKLOADS["unet_bf16"][1]]),
}


def workload_of(layer_name: str) -> str:
    for wname, (_, ls) in list(WORKLOADS.items()) + list(EXTRA_WORKLOADS.items()):
        if any(l.name == layer_name for l in ls):
            return wname
    raise KeyError(layer_name)


# ---------------------------------------------------------------- quantisation
def bf16_bits_from_f32(a32: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (RNE) and return the 16-bit patterns.

    The inputs drawn here are finite, so no NaN handling is needed.
    """
    u = np.ascontiguousarray(a32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


class Tensor:
    """A quantised tensor: storage bits (numpy) plus the exact float64 values."""

    def __init__(self, dtype: str, storage: np.ndarray):
        self.dtype = dtype
        self.storage = storage          # float32, float16, or uint16 (bf16 bits)

    @staticmethod
    def quantise(a64: np.ndarray, dtype: str) -> "Tensor":
        if dtype == "f32":
            return Tensor(dtype, a64.astype(np.float32))
        if dtype == "f16":
            return Tensor(dtype, a64.astype(np.float16))
        if dtype == "bf16":
            return Tensor(dtype, bf16_bits_from_f32(a64.astype(np.float32)))
        raise ValueError(dtype)

    @property
    def shape(self):
        return self.storage.shape

    def f64(self) -> np.ndarray:
        if self.dtype == "bf16":
            return bf16_bits_to_f64(self.storage)
        return self.storage.astype(np.float64)

    def torch(self, device="cpu"):
        import torch
        t = torch.from_numpy(np.ascontiguousarray(self.storage))
        if self.dtype == "bf16":
            t = t.view(torch.bfloat16)
        return t.to(device)


def _sample(rng: np.random.Generator, dist: str, shape) -> np.ndarray:
    if dist == "U01":
        return rng.uniform(0.0, 1.0, size=shape)
    if dist == "U11":
        return rng.uniform(-1.0, 1.0, size=shape)
    if dist == "N01":
        return rng.standard_normal(size=shape)
    if dist.startswith("U0."):
        a = float(dist[1:])
        return rng.uniform(-a, a, size=shape)
    raise ValueError(dist)


def _draw(rng: np.random.Generator, layer: Layer):
    x = _sample(rng, layer.x_dist, layer.x_shape)
    w = _sample(rng, layer.w_dist, layer.w_shape) / math.sqrt(layer.fan_in)
    if layer.b_dist == "zero":
        b = np.zeros(layer.C_out)
    else:
        b = _sample(rng, layer.b_dist, (layer.C_out,))
    return x, w, b


def make_inputs(layer: Layer, seed: Optional[int] = None):
    """Quantised (x, w, b) for ``layer``.

    With ``seed=None`` the layer is one of the five workloads and its values
    come from that workload's generator, drawn in workload order (so a layer's
    values do not depend on which other layers a caller asks for).  With an
    explicit seed, the layer (any shape) gets its own generator.
    """
    if seed is None:
        wname = workload_of(layer.name)
        wseed, layers = {**WORKLOADS, **EXTRA_WORKLOADS}[wname]
        rng = np.random.default_rng(wseed)
        for l in layers:
            if l.name == layer.name:
                x, w, b = _draw(rng, l)
                break
            # advance the generator exactly as drawing this layer would
            _draw(rng, l)
    else:
        rng = np.random.default_rng(seed)
        x, w, b = _draw(rng, layer)
    d = layer.dtype
    return Tensor.quantise(x, d), Tensor.quantise(w, d), Tensor.quantise(b, d)
