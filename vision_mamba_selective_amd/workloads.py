"""Seeded synthetic inputs for the selective scan.

This module only draws and rounds numbers. It holds none of the scan's
arithmetic, so both the HIP path and the fp64 oracle can be fed from it
without sharing any of the method.

Workloads stand in for the shapes the source pages discuss (no image data or
trained weights exist here):

* "Vision Mamba Guide: Efficient Bidirectional SSM & VMamba" (aifetchly blog),
  section "The Quadratic Bottleneck in Vision Transformers": 224x224, 1024x1024
  and 2048x2048 images at 16x16 patches give 196, 4,096 and 16,384 patches;
  section "1. Patch Tokenization and Position Embedding" prepends one class
  token, so a Vim sequence has 197, 4,097 or 16,385 tokens.
* Same page, section "Empirical Benchmarks & Performance Analysis", table
  "Classification & High-Resolution Benchmark Comparison": Vim-S at 1248x1248
  (78 x 78 patches of 16 pixels plus the class token: 6,085 tokens). The page
  gives no batch size; batch 8 matches the 1024x1024 workload.
* Same page, section "VMamba: 2D Selective Scan (SS2D) and Cross-Scan
  Traversal": a feature grid unrolled in four orders (64x64 here).
* Same page, section "PyTorch Implementation of the Bidirectional Vision Mamba
  Block": A is initialised from log(1..d_state), i.e. A[d, n] = -(n+1), and the
  state size defaults to 16.

Draw order (one ``numpy.random.default_rng(seed)`` stream, PCG64):
  1. u, z, delta-noise, each standard normal of shape [batch, dim, L]
     (float32 draws); delta_raw = 0.5 * noise.
  2. B, then C: standard normal, [batch, dstate, L] (shared by the directions)
     or [batch, ndir, dstate, L] (one per direction, in that direction's scan
     order).
  3. For each direction k: dt_k = exp(U(log lo, log hi)) per channel, and
     dt_bias_k = log(expm1(dt_k)) in float64, rounded to float32 (the inverse
     of softplus, so that softplus(dt_bias_k) = dt_k).
  4. A_k[d, n] = -(n+1), D_k[d] = 1 (float32), unless a variant asks for
     random A (A = -U(0.1, 20)) or random D (N(0, 1)).
Activations are rounded to the workload dtype with round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: its shapes, dtype and input distribution."""

    name: str
    kind: str            # "vim" (forward + backward) or "cross4" (VMamba four orders)
    batch: int
    dim: int             # d_inner, the number of channels
    dstate: int
    seqlen: int          # tokens per direction
    dtype: str           # F32 or BF16: dtype of u, delta, z, B, C and y
    dt_min: float
    dt_max: float
    H: int = 0           # grid height (cross4 only)
    W: int = 0           # grid width (cross4 only)
    gate: bool = True    # multiply the merged output by silu(z)
    seed: int = 0

    @property
    def ndir(self) -> int:
        return 2 if self.kind == "vim" else 4

    @property
    def tokens_channels(self) -> int:
        return self.batch * self.dim * self.seqlen

    @property
    def state_updates(self) -> int:
        return self.tokens_channels * self.ndir * self.dstate

    @property
    def act_bytes(self) -> int:
        return 2 if self.dtype == BF16 else 4

    def algorithmic_bytes(self) -> int:
        """Bytes the scan must move at minimum: read u, delta_raw, (z), B, C and
        the per-direction parameters once, write y once."""
        e = self.act_bytes
        tc = self.tokens_channels
        n_act = 3 + (1 if self.gate else 0)  # u, delta, y (+ z)
        bc_per = self.ndir if self.kind == "cross4" else 1
        bc = 2 * self.batch * bc_per * self.dstate * self.seqlen * e
        params = self.ndir * self.dim * (self.dstate + 2) * 4
        return n_act * tc * e + bc + params

    def grad_algorithmic_bytes(self) -> int:
        """Bytes the gradient must move at minimum (Vim): read u, delta_raw,
        (z), dy, B, C and the parameters once; write du, ddelta, (dz) in the
        activation dtype, dB and dC in fp32 and the parameter gradients
        once."""
        e = self.act_bytes
        tc = self.tokens_channels
        g = 1 if self.gate else 0
        bc = self.batch * self.dstate * self.seqlen
        params = self.ndir * self.dim * (self.dstate + 2) * 4
        reads = (3 + g) * tc * e + 2 * bc * e + params
        writes = (2 + g) * tc * e + 2 * bc * 4 + params
        return reads + writes

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _vim(name, batch, seqlen, dim, dtype, dt_min, dt_max, seed):
    return Workload(name=name, kind="vim", batch=batch, dim=dim, dstate=16,
                    seqlen=seqlen, dtype=dtype, dt_min=dt_min, dt_max=dt_max,
                    seed=seed)


#: The workloads. Index 2 (Vim-S at 1024^2) is the throughput headline; index
#: 5 (Vim-S at 1248^2) is the resolution of the guide's memory comparison.
WORKLOADS = [
    _vim("vim_ti_224_f32", 1, 197, 384, F32, 1e-3, 1e-1, 1000),
    _vim("vim_s_224_bf16", 64, 197, 768, BF16, 1e-3, 1e-1, 1001),
    _vim("vim_s_1024_bf16", 8, 4097, 768, BF16, 1e-3, 1e-1, 1002),
    Workload(name="vmamba_cross4_64x64_f32", kind="cross4", batch=8, dim=384,
             dstate=16, seqlen=64 * 64, dtype=F32, dt_min=1e-3, dt_max=1e-1,
             H=64, W=64, gate=False, seed=1003),
    _vim("vim_b_2048_bf16", 2, 16385, 1536, BF16, 1e-4, 1e-1, 1004),
    _vim("vim_s_1248_bf16", 8, (1248 // 16) ** 2 + 1, 768, BF16, 1e-3, 1e-1, 1005),
]

HEADLINE = 2


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even) and return
    them as float32. Inputs must be finite."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return (b.astype(np.uint32) << 16).view(np.float32)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Bit patterns (uint16) of float32 values that are already bf16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    if np.any(bits & 0xFFFF):
        raise ValueError("values are not bf16-representable")
    return (bits >> 16).astype(np.uint16)


@dataclasses.dataclass
class Inputs:
    """Host arrays for one call. Activations are float32 arrays that hold
    exactly the values given to the GPU (bf16-representable for bf16
    workloads)."""

    wl: Workload
    u: np.ndarray
    delta: np.ndarray
    z: Optional[np.ndarray]
    B: np.ndarray
    C: np.ndarray
    A: np.ndarray        # [ndir, dim, dstate] float32
    D: np.ndarray        # [ndir, dim] float32
    dt_bias: np.ndarray  # [ndir, dim] float32


def make_inputs(wl: Workload, seed: Optional[int] = None, *, random_A: bool = False,
                random_D: bool = False, delta_scale: float = 0.5) -> Inputs:
    """Draw the inputs of ``wl`` with the documented recipe."""
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    shape = (wl.batch, wl.dim, wl.seqlen)
    u = rng.standard_normal(shape, dtype=np.float32)
    z = rng.standard_normal(shape, dtype=np.float32)
    delta = rng.standard_normal(shape, dtype=np.float32)
    delta *= np.float32(delta_scale)
    if wl.kind == "cross4":
        bc_shape = (wl.batch, wl.ndir, wl.dstate, wl.seqlen)
    else:
        bc_shape = (wl.batch, wl.dstate, wl.seqlen)
    B = rng.standard_normal(bc_shape, dtype=np.float32)
    C = rng.standard_normal(bc_shape, dtype=np.float32)
    dt_bias = np.empty((wl.ndir, wl.dim), np.float32)
    for k in range(wl.ndir):
        dt = np.exp(rng.uniform(math.log(wl.dt_min), math.log(wl.dt_max), wl.dim))
        dt_bias[k] = np.log(np.expm1(dt)).astype(np.float32)
    if random_A:
        A = -rng.uniform(0.1, 20.0, (wl.ndir, wl.dim, wl.dstate)).astype(np.float32)
    else:
        A = np.broadcast_to(-(np.arange(wl.dstate, dtype=np.float32) + 1),
                            (wl.ndir, wl.dim, wl.dstate)).copy()
    if random_D:
        D = rng.standard_normal((wl.ndir, wl.dim)).astype(np.float32)
    else:
        D = np.ones((wl.ndir, wl.dim), np.float32)
    if wl.dtype == BF16:
        u, z, delta, B, C = (round_bf16(a) for a in (u, z, delta, B, C))
    return Inputs(wl=wl, u=u, delta=delta, z=z if wl.gate else None, B=B, C=C,
                  A=A, D=D, dt_bias=dt_bias)


def channel_subset(inp: Inputs, batches, channels) -> Inputs:
    """The same inputs restricted to the given batch rows and channels. The
    scan of one (batch, channel) pair depends only on that pair's row of u,
    delta and z, its batch's B and C, and its channel's parameters, so the
    outputs of the subset equal the matching outputs of the full problem."""
    bi = np.asarray(batches)
    ci = np.asarray(channels)
    sub = lambda a: None if a is None else np.ascontiguousarray(a[bi][:, ci])
    wl = inp.wl.with_(batch=len(bi), dim=len(ci))
    return Inputs(wl=wl, u=sub(inp.u), delta=sub(inp.delta), z=sub(inp.z),
                  B=np.ascontiguousarray(inp.B[bi]), C=np.ascontiguousarray(inp.C[bi]),
                  A=np.ascontiguousarray(inp.A[:, ci]), D=np.ascontiguousarray(inp.D[:, ci]),
                  dt_bias=np.ascontiguousarray(inp.dt_bias[:, ci]))
