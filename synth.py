"""Seeded synthetic inputs for the fused GEMM + bias/activation workloads.

This module holds the workload table and the seeded random draws only -- none
of the method's arithmetic.  Tests and the benchmark use it to create the
device buffers that both the HIP library and the CPU oracle then read (the
oracle reads the device values back; it never regenerates them).

Draw order per workload: A, B, bias, each rounded to its storage dtype with
round-to-nearest-even (torch's cast).  fp8-e4m3 operands are drawn in fp32,
then quantised per tensor: s = amax|x| / 448, code = e4m3(clamp(x / s, +-448)),
so that x ~= s * decode(code); s travels as an fp32 device scalar.

"N(0, v)" in a workload's description is read as mean 0 and *variance* v.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
               "e4m3": torch.float8_e4m3fn, "mxf8": torch.float8_e4m3fn}
ELEM_SIZE = {"f32": 4, "f16": 2, "bf16": 2, "e4m3": 1, "mxf8": 1}
E4M3_EMAX = 8   # exponent of E4M3's largest power of two (448 = 1.75 * 2^8)
E4M3_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class Workload:
    key: str
    name: str
    m: int
    n: int
    k: int
    in_dtype: str         # dtype of A and B
    out_dtype: str        # dtype of D (and of the bias)
    epilog: str           # none | bias | relu_bias | relu_aux_bias | gelu_bias
                          # | gelu_aux_bias | drelu | dgelu | drelu_bgrad | dgelu_bgrad
    axis: str             # row: bias has m values; col: bias has n values
    op_b: int             # 0: B is k x n row-major; 1: B is n x k (Linear weight)
    seed: int
    a_dist: tuple         # ("normal", variance) | ("uniform", lo, hi)
    b_dist: tuple
    bias_dist: tuple

    @property
    def flops(self) -> float:
        return 2.0 * self.m * self.n * self.k

    def algorithmic_bytes(self) -> int:
        """A, B, bias and D read or written once, plus the aux buffer: the
        1-bit mask (written by relu_aux_bias, read by drelu) or the m x n
        pre-activation in D's dtype (written by gelu_aux_bias, read by dgelu)."""
        ea, eo = ELEM_SIZE[self.in_dtype], ELEM_SIZE[self.out_dtype]
        # the bias is read, or (bias-gradient epilogues) written, once
        biased = self.epilog not in ("none", "drelu", "dgelu")
        nb = (self.m if self.axis == "row" else self.n) * eo if biased else 0
        aux = 0
        if self.epilog in ("relu_aux_bias", "drelu", "drelu_bgrad"):
            aux = self.m * (((self.n + 127) // 128) * 16)
        elif self.epilog in ("gelu_aux_bias", "dgelu", "dgelu_bgrad"):
            aux = self.m * self.n * eo
        scales = 8 if self.in_dtype == "e4m3" else 0
        if self.in_dtype == "mxf8":   # one byte per 32 K values of every row of A and column of B
            scales = (self.m + self.n) * ((self.k + 31) // 32)
        return (self.m * self.k + self.k * self.n) * ea + nb + self.m * self.n * eo + aux + scales


# The pages' workloads: the nvmath example shape (1024, 512, 2048) with an
# (m,1) bias; the Linear(4096,4096)+GELU module at batch 16; the H200
# benchmark shape 65536x16384 by 16384x8192; a square 8192^3 case for the
# aux-mask epilogue; and a tiny fp32 case.
WORKLOADS = {
    "C1": Workload("C1", "fp32 GEMM+BIAS 128x64x256", 128, 64, 256, "f32", "f32", "bias", "row", 0,
                   1001, ("normal", 1.0), ("normal", 1.0), ("normal", 1.0)),
    "C2": Workload("C2", "fp16 GEMM+BIAS 1024x512x2048", 1024, 512, 2048, "f16", "f16", "bias", "row", 0,
                   1002, ("normal", 1.0), ("normal", 1.0), ("normal", 1.0)),
    "C3": Workload("C3", "fp16 Linear 16x4096x4096 GELU_BIAS", 16, 4096, 4096, "f16", "f16", "gelu_bias",
                   "col", 1, 1003, ("normal", 1.0), ("uniform", -1 / 64, 1 / 64),
                   ("uniform", -1 / 64, 1 / 64)),
    "C4": Workload("C4", "bf16 RELU_AUX_BIAS 8192x8192x8192", 8192, 8192, 8192, "bf16", "bf16",
                   "relu_aux_bias", "row", 0, 1004, ("normal", 1 / math.sqrt(8192)),
                   ("normal", 1 / math.sqrt(8192)), ("normal", 0.1)),
    "C5a": Workload("C5a", "bf16 RELU_BIAS 65536x8192x16384", 65536, 8192, 16384, "bf16", "bf16",
                    "relu_bias", "row", 0, 1005, ("normal", 1 / math.sqrt(16384)),
                    ("normal", 1 / math.sqrt(16384)), ("normal", 0.1)),
    "C5b": Workload("C5b", "fp8-e4m3 RELU_BIAS 65536x8192x16384", 65536, 8192, 16384, "e4m3", "bf16",
                    "relu_bias", "row", 0, 1005, ("normal", 1 / math.sqrt(16384)),
                    ("normal", 1 / math.sqrt(16384)), ("normal", 0.1)),
    # block-scaled fp8 (MX: one E8M0 scale per 32 K values) at the H200 shape
    "F2a": Workload("F2a", "mxfp8 RELU_BIAS 65536x8192x16384", 65536, 8192, 16384, "mxf8", "bf16",
                    "relu_bias", "row", 0, 1010, ("normal", 1 / math.sqrt(16384)),
                    ("normal", 1 / math.sqrt(16384)), ("normal", 0.1)),
    # training-side epilogues at the square 8192^3 shape: the GELU forward
    # that keeps its pre-activation, and the two backward products (the
    # upstream gradient times the next layer's weight) scaled by GELU' or by
    # ReLU' from the stored aux buffer
    "F1a": Workload("F1a", "bf16 GELU_AUX_BIAS 8192x8192x8192", 8192, 8192, 8192, "bf16", "bf16",
                    "gelu_aux_bias", "row", 0, 1006, ("normal", 1 / math.sqrt(8192)),
                    ("normal", 1 / math.sqrt(8192)), ("normal", 0.1)),
    "F1b": Workload("F1b", "bf16 DGELU 8192x8192x8192", 8192, 8192, 8192, "bf16", "bf16",
                    "dgelu", "row", 0, 1007, ("normal", 1 / math.sqrt(8192)),
                    ("normal", 1 / math.sqrt(8192)), ("normal", 0.1)),
    "F1c": Workload("F1c", "bf16 DRELU 8192x8192x8192", 8192, 8192, 8192, "bf16", "bf16",
                    "drelu", "row", 0, 1008, ("normal", 1 / math.sqrt(8192)),
                    ("normal", 1 / math.sqrt(8192)), ("normal", 0.1)),
    # the backward of a Linear layer's GELU with its bias gradient: the bias
    # was added to every row, so its gradient sums the columns
    "F1d": Workload("F1d", "bf16 DGELU_BGRAD 8192x8192x8192", 8192, 8192, 8192, "bf16", "bf16",
                    "dgelu_bgrad", "col", 0, 1009, ("normal", 1 / math.sqrt(8192)),
                    ("normal", 1 / math.sqrt(8192)), ("normal", 0.1)),
}

# variance of the stored pre-activation a backward workload reads: that of
# the forward's A*B (1 with the variances above) plus its bias (0.1)
AUX_PRE_VARIANCE = 1.1


def scaled(w: Workload, m: Optional[int] = None, n: Optional[int] = None,
           k: Optional[int] = None, **kw) -> Workload:
    """Same recipe at another size (for parity cases the oracle can finish)."""
    return dataclasses.replace(w, m=m or w.m, n=n or w.n, k=k or w.k, **kw)


def _draw(gen: torch.Generator, shape, dist, device) -> torch.Tensor:
    if dist[0] == "normal":
        return torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * math.sqrt(dist[1])
    if dist[0] == "uniform":
        lo, hi = dist[1], dist[2]
        return torch.rand(shape, generator=gen, device=device, dtype=torch.float32) * (hi - lo) + lo
    if dist[0] == "int":
        lo, hi = dist[1], dist[2]
        return torch.randint(lo, hi + 1, shape, generator=gen, device=device).to(torch.float32)
    if dist[0] == "zeros":
        return torch.zeros(shape, device=device, dtype=torch.float32)
    raise ValueError(dist)


def quantise_e4m3(x: torch.Tensor):
    """Per-tensor fp8 quantisation: returns (codes, scale) with x ~= scale*codes."""
    amax = x.abs().max().to(torch.float32)
    s = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    q = torch.clamp(x / s, -E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return q, s.reshape(1).to(torch.float32)


def mx_scale_ld(k: int) -> int:
    """Row stride in bytes of an MX block-scale array: ceil(k/32) scales,
    rounded up to 16 bytes."""
    return ((k + 31) // 32 + 15) // 16 * 16


def quantise_mx(x: torch.Tensor):
    """MX block quantisation along the last axis (OCP Microscaling, E4M3
    elements): each run of 32 values shares the E8M0 scale 2^(e - 127) with
    e - 127 = floor(log2(amax of the run)) - 8 (8 being E4M3's largest
    exponent); the elements are x / scale rounded to E4M3, saturating at 448.
    An all-zero run gets e = 127.  Returns (codes as float8_e4m3fn, scales as
    uint8 rows of mx_scale_ld(k) bytes, padding 127)."""
    rows, k = x.shape
    kb = (k + 31) // 32
    xp = torch.zeros((rows, kb * 32), dtype=torch.float32, device=x.device)
    xp[:, :k] = x
    blocks = xp.reshape(rows, kb, 32)
    amax = blocks.abs().amax(dim=2)
    e = torch.where(amax > 0, torch.floor(torch.log2(torch.where(amax > 0, amax, torch.ones_like(amax)))) - E4M3_EMAX,
                    torch.zeros_like(amax))
    e = torch.clamp(e, -127, 127)
    q = torch.clamp(blocks / torch.exp2(e)[:, :, None], -E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    codes = q.reshape(rows, kb * 32)[:, :k].contiguous()
    scales = torch.full((rows, mx_scale_ld(k)), 127, dtype=torch.uint8, device=x.device)
    scales[:, :kb] = (e + 127).to(torch.uint8)
    return codes, scales


@dataclasses.dataclass
class Inputs:
    A: torch.Tensor
    B: torch.Tensor
    bias: Optional[torch.Tensor]
    scale_a: Optional[torch.Tensor]
    scale_b: Optional[torch.Tensor]
    mx_a: Optional[torch.Tensor] = None   # MX block scales of A's rows (m x mx_scale_ld(k), uint8)
    mx_b: Optional[torch.Tensor] = None   # of B's columns (n x mx_scale_ld(k), uint8)


def make_inputs(w: Workload, device="cpu", seed: Optional[int] = None,
                a_dist=None, b_dist=None, bias_dist=None) -> Inputs:
    """Draw A (m x k), B (k x n, or n x k when op_b=1) and the bias, in that
    order, from torch's generator on `device` seeded with the workload seed."""
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed if seed is None else seed)
    a = _draw(gen, (w.m, w.k), a_dist or w.a_dist, device)
    b = _draw(gen, (w.n, w.k) if w.op_b else (w.k, w.n), b_dist or w.b_dist, device)
    nbias = w.m if w.axis == "row" else w.n
    bias = _draw(gen, (nbias,), bias_dist or w.bias_dist, device)
    sa = sb = None
    mxa = mxb = None
    if w.in_dtype == "mxf8":
        A, mxa = quantise_mx(a)
        del a
        # B's scales follow its columns' K runs, whichever layout B has
        if w.op_b:
            B, mxb = quantise_mx(b)
        else:
            Bt, mxb = quantise_mx(b.t().contiguous())
            B = Bt.t().contiguous()
            del Bt
        del b
    elif w.in_dtype == "e4m3":
        A, sa = quantise_e4m3(a)
        del a
        B, sb = quantise_e4m3(b)
        del b
    else:
        A = a.to(TORCH_DTYPE[w.in_dtype])
        del a
        B = b.to(TORCH_DTYPE[w.in_dtype])
        del b
    bias = bias.to(TORCH_DTYPE[w.out_dtype])
    if w.axis == "row":
        bias = bias.reshape(w.m, 1)   # the (m,1) form of the nvmath example
    return Inputs(A.contiguous(), B.contiguous(), bias.contiguous(), sa, sb, mxa, mxb)


def aux_ld_words(n: int) -> int:
    """Row stride, in 32-bit words, of the packed ReLU mask: rows padded to
    128 bits so every row starts 16-byte aligned."""
    return ((n + 127) // 128) * 4


def aux_ld_elems(n: int) -> int:
    """Row stride, in elements, of the pre-activation aux matrix: rows padded
    to 128 elements."""
    return ((n + 127) // 128) * 128


def make_aux(w: Workload, device="cpu", seed: Optional[int] = None) -> torch.Tensor:
    """The aux input of a backward workload, drawn after nothing else from a
    generator seeded with seed + 1: for drelu, mask words with independent
    fair bits (m x aux_ld_words); for dgelu, a pre-activation matrix
    ~ N(0, AUX_PRE_VARIANCE) in D's dtype (m x aux_ld_elems)."""
    gen = torch.Generator(device=device)
    gen.manual_seed((w.seed if seed is None else seed) + 1)
    if w.epilog in ("drelu", "drelu_bgrad"):
        t = torch.randint(0, 2 ** 32, (w.m, aux_ld_words(w.n)), generator=gen, device=device,
                          dtype=torch.int64)
        return (t - 2 ** 31).to(torch.int32)
    if w.epilog in ("dgelu", "dgelu_bgrad"):
        x = _draw(gen, (w.m, aux_ld_elems(w.n)), ("normal", AUX_PRE_VARIANCE), device)
        return x.to(TORCH_DTYPE[w.out_dtype])
    raise ValueError(f"{w.epilog} reads no aux input")
