"""Seeded synthetic inputs for In-Place Activated BatchNorm.

This module only draws random tensors and rounds them to the storage dtype.
It holds none of the method's arithmetic, so that the fp64 oracle and the HIP
path can both consume the very same input bits.

Workloads: the pages train ResNeXt / WideResNet bodies on ImageNet-1k and
DeepLabV3 heads on Cityscapes and Mapillary Vistas (page 3, section 4
"Experiments").  Those datasets are not available; the five shapes below stand
in for activations of such networks: a ResNet mid-stage map, a segmentation-scale
feature map, a numerically hard channel mix, and a many-channel backbone tail.

Recipe (all configurations):
  * numpy PCG64 generator, seed 1000 + configuration index (1..5);
  * draw order: per-channel location mu_c, per-channel scale s_c, gamma sign,
    gamma magnitude, beta_c, then x, then dy (each only when the recipe uses it);
  * x and dy are drawn in logical NCHW order as fp64, permuted to the storage
    layout, then rounded to the storage dtype (fp32 by numpy's RNE cast; bf16 by
    round-to-nearest-even on the fp32 bit pattern; fp16 by numpy's RNE cast of
    the fp32 value);
  * "N(a, b)" means mean a and *variance* b;
  * running statistics start at mean 0, variance 1.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

LAYOUTS = ("NCHW", "NHWC")
DTYPES = ("f32", "bf16", "f16")
ACTS = ("identity", "leaky_relu", "elu")


@dataclasses.dataclass(frozen=True)
class Recipe:
    """Distributions for one workload.  Each tuple is (kind, a, b)."""
    mu: tuple = ("const", 0.0, 0.0)          # per-channel location of x
    scale: tuple = ("const", 1.0, 1.0)       # per-channel std of x: const/uniform/log10uniform
    gamma: tuple = ("uniform", 0.5, 1.5)     # magnitude of gamma
    gamma_signed: bool = False               # random sign on gamma
    beta_var: float = 0.1                    # beta ~ N(0, beta_var)
    dy_var: float = 1.0                      # dy ~ N(0, dy_var)


@dataclasses.dataclass(frozen=True)
class Workload:
    index: int
    name: str
    N: int
    C: int
    H: int
    W: int
    layout: str
    dtype: str
    act: str
    act_param: float
    eps: float
    momentum: float
    recipe: Recipe

    @property
    def numel(self) -> int:
        return self.N * self.C * self.H * self.W

    @property
    def m(self) -> int:
        return self.N * self.H * self.W

    @property
    def esize(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def storage_bytes(self) -> int:
        return self.numel * self.esize

    def with_shape(self, N: int, C: int, H: int, W: int) -> "Workload":
        return dataclasses.replace(self, N=N, C=C, H=H, W=W)


CONFIGS = [
    Workload(1, "tiny_nchw_f32_leaky", 2, 4, 8, 8, "NCHW", "f32", "leaky_relu", 0.01,
             1e-5, 0.1,
             Recipe(mu=("uniform", -1.0, 1.0), scale=("uniform", 0.5, 2.0),
                    gamma=("uniform", 0.5, 1.5), gamma_signed=True, beta_var=0.1, dy_var=1.0)),
    Workload(2, "resnet_mid_nchw_f32_leaky", 32, 256, 56, 56, "NCHW", "f32", "leaky_relu", 0.01,
             1e-5, 0.1,
             Recipe(mu=("uniform", -0.5, 0.5), gamma=("uniform", 0.5, 1.5),
                    beta_var=0.1, dy_var=1.0)),
    Workload(3, "segmap_nhwc_bf16_leaky", 2, 256, 512, 512, "NHWC", "bf16", "leaky_relu", 0.01,
             1e-5, 0.1,
             Recipe(gamma=("uniform", 0.5, 1.5), beta_var=0.1, dy_var=1e-2)),
    Workload(4, "stress_nchw_f32_elu", 16, 512, 28, 28, "NCHW", "f32", "elu", 1.0,
             1e-5, 0.1,
             Recipe(mu=("uniform", -5.0, 5.0), scale=("log10uniform", -2.0, 2.0),
                    gamma=("uniform", 0.1, 2.0), gamma_signed=True, beta_var=0.5, dy_var=1.0)),
    Workload(5, "tail_nhwc_bf16_leaky", 64, 2048, 7, 7, "NHWC", "bf16", "leaky_relu", 0.01,
             1e-5, 0.1,
             Recipe(gamma=("uniform", 0.5, 1.5), beta_var=0.1, dy_var=1.0)),
]


def config(index: int) -> Workload:
    """Workload by its 1-based index."""
    return CONFIGS[index - 1]


# --------------------------------------------------------------------------------------
# storage rounding (input side only)

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16), round to nearest even, NaN kept quiet."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = np.isnan(a)
    rounded = np.where(nan, (u >> 16) | 0x40, rounded)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_storage(x_nchw: np.ndarray, layout: str, dtype: str) -> np.ndarray:
    """fp64 logical-NCHW array -> storage array (float32, or uint16 bf16 / fp16 bits)
    in `layout`."""
    if layout == "NHWC":
        x_nchw = np.transpose(x_nchw, (0, 2, 3, 1))
    f32 = np.ascontiguousarray(x_nchw, dtype=np.float32)
    if dtype == "f32":
        return f32
    if dtype == "bf16":
        return f32_to_bf16_bits(f32)
    if dtype == "f16":
        with np.errstate(over="ignore"):
            return f32.astype(np.float16).view(np.uint16)
    raise ValueError(dtype)


def from_storage(s: np.ndarray, N: int, C: int, H: int, W: int, layout: str, dtype: str) -> np.ndarray:
    """storage array -> fp64 logical-NCHW array (exact upcast)."""
    if dtype == "bf16":
        f = bf16_bits_to_f32(s.reshape(-1))
    elif dtype == "f16":
        f = np.ascontiguousarray(s, dtype=np.uint16).reshape(-1).view(np.float16).astype(np.float32)
    else:
        f = np.ascontiguousarray(s, dtype=np.float32).reshape(-1)
    if layout == "NCHW":
        return f.reshape(N, C, H, W).astype(np.float64)
    return np.ascontiguousarray(np.transpose(f.reshape(N, H, W, C), (0, 3, 1, 2))).astype(np.float64)


# --------------------------------------------------------------------------------------
# draws

def _draw_vec(rng: np.random.Generator, spec: tuple, C: int) -> np.ndarray:
    kind, a, b = spec
    if kind == "const":
        return np.full(C, a, dtype=np.float64)
    if kind == "uniform":
        return rng.uniform(a, b, size=C)
    if kind == "log10uniform":
        return 10.0 ** rng.uniform(a, b, size=C)
    raise ValueError(kind)


@dataclasses.dataclass
class Inputs:
    wl: Workload
    x: np.ndarray          # storage array (float32 or uint16 bits), in wl.layout
    dy: np.ndarray         # storage array, in wl.layout
    gamma: np.ndarray      # float32 [C]
    beta: np.ndarray       # float32 [C]
    running_mean: np.ndarray  # float32 [C]
    running_var: np.ndarray   # float32 [C]


def make_inputs(wl: Workload, seed: Optional[int] = None, with_dy: bool = True) -> Inputs:
    """Draw one seeded input set for workload `wl` (its own shape)."""
    rng = np.random.Generator(np.random.PCG64(1000 + wl.index if seed is None else seed))
    r = wl.recipe
    C = wl.C
    mu = _draw_vec(rng, r.mu, C)
    sc = _draw_vec(rng, r.scale, C)
    sign = (rng.integers(0, 2, size=C) * 2 - 1).astype(np.float64) if r.gamma_signed else np.ones(C)
    gmag = _draw_vec(rng, r.gamma, C)
    beta = rng.normal(0.0, np.sqrt(r.beta_var), size=C)
    gamma = sign * gmag
    shape = (wl.N, C, wl.H, wl.W)
    x = rng.standard_normal(size=shape)
    x *= sc[None, :, None, None]
    x += mu[None, :, None, None]
    xs = to_storage(x, wl.layout, wl.dtype)
    del x
    if with_dy:
        dy = rng.normal(0.0, np.sqrt(r.dy_var), size=shape)
        dys = to_storage(dy, wl.layout, wl.dtype)
        del dy
    else:
        dys = None
    return Inputs(wl=wl, x=xs, dy=dys,
                  gamma=gamma.astype(np.float32), beta=beta.astype(np.float32),
                  running_mean=np.zeros(C, np.float32), running_var=np.ones(C, np.float32))


@dataclasses.dataclass
class DeviceInputs:
    """Inputs drawn directly in device memory, for tensors too large to build on the
    host.  x and dy are torch tensors in the storage layout and dtype; the
    per-channel vectors are float32 numpy arrays."""
    wl: Workload
    x: object
    dy: object
    gamma: np.ndarray
    beta: np.ndarray
    running_mean: np.ndarray
    running_var: np.ndarray


def make_device_inputs(wl: Workload, seed: int, device="cuda") -> DeviceInputs:
    """The workload's recipe drawn on the device: per-channel parameters from numpy
    PCG64(seed) as in make_inputs (same draw order); x and dy from torch's
    device generator seeded with `seed`, drawn in the storage layout in fp32 and
    rounded to the storage dtype by torch's (nearest-even) cast."""
    import torch
    rng = np.random.Generator(np.random.PCG64(seed))
    r = wl.recipe
    C = wl.C
    mu = _draw_vec(rng, r.mu, C)
    sc = _draw_vec(rng, r.scale, C)
    sign = (rng.integers(0, 2, size=C) * 2 - 1).astype(np.float64) if r.gamma_signed else np.ones(C)
    gmag = _draw_vec(rng, r.gamma, C)
    beta = rng.normal(0.0, np.sqrt(r.beta_var), size=C)
    shape = (wl.N, C, wl.H, wl.W) if wl.layout == "NCHW" else (wl.N, wl.H, wl.W, C)
    bshape = (1, C, 1, 1) if wl.layout == "NCHW" else (1, 1, 1, C)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    dt = storage_torch_dtype(wl.dtype)
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    x.mul_(torch.tensor(sc, dtype=torch.float32, device=device).view(bshape))
    x.add_(torch.tensor(mu, dtype=torch.float32, device=device).view(bshape))
    x = x.to(dt)
    dy = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    dy.mul_(float(np.sqrt(r.dy_var)))
    dy = dy.to(dt)
    return DeviceInputs(wl=wl, x=x, dy=dy, gamma=(sign * gmag).astype(np.float32),
                        beta=beta.astype(np.float32), running_mean=np.zeros(C, np.float32),
                        running_var=np.ones(C, np.float32))


def device_channel(t, wl: Workload, c: int) -> np.ndarray:
    """Channel c of a device storage tensor as an fp64 [N, 1, H, W] host array."""
    import torch
    if wl.layout == "NCHW":
        v = t[:, c:c + 1, :, :]
    else:
        v = t[:, :, :, c].unsqueeze(1)
    return v.to(torch.float32).cpu().numpy().astype(np.float64)


def storage_torch_dtype(dtype: str):
    """torch dtype used to hold the storage bits (bf16 bits travel as torch.bfloat16,
    fp16 bits as torch.float16)."""
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]


def to_torch(a: np.ndarray, dtype: str):
    """numpy storage array -> CPU torch tensor holding the same bits."""
    import torch
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16)


def from_torch(t, dtype: str) -> np.ndarray:
    """CPU torch tensor -> numpy storage array with the same bits."""
    import torch
    t = t.detach().cpu().contiguous()
    if dtype == "f32":
        return t.numpy().astype(np.float32, copy=False)
    return t.view(torch.int16).numpy().view(np.uint16)
