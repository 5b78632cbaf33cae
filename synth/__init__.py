"""Seeded synthetic inputs for the fused DiT-block epilogues.

This module only draws random tensors; it holds none of the epilogues'
arithmetic. Both the GPU path and the CPU oracle are fed the exact bytes it
returns, so a parity test compares the two on identical inputs.

Every tensor is drawn on the CPU with ``torch.Generator().manual_seed(seed)``
as float32 ``randn * std + mean`` and rounded to bfloat16 by torch (round to
nearest even). Shapes and distributions follow the Qwen-Image and FLUX.2
workloads the pages measure (hidden 3072, 24 heads x 128, 512 text + 4096
image tokens; FLUX.2 single-block rows of 6144 attention + 18432 MLP
columns). No dataset, checkpoint or prompt is involved.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

__all__ = [
    "bf16_bits",
    "NormModulateInputs",
    "ScaleResidualInputs",
    "QkvInputs",
    "BiasMulAddInputs",
    "TokenCatInputs",
    "norm_modulate_inputs",
    "scale_residual_inputs",
    "qkv_inputs",
    "bias_mul_add_inputs",
    "token_cat_inputs",
    "rope_tables",
    "fp4_global_scale",
]


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _normal_bf16(g: torch.Generator, shape, mean: float = 0.0, std: float = 1.0) -> torch.Tensor:
    t = torch.randn(*shape, generator=g, dtype=torch.float32)
    return (t * std + mean).to(torch.bfloat16).contiguous()


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bfloat16 bit patterns of a CPU tensor as a uint16 numpy array."""
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


@dataclass
class NormModulateInputs:
    x: torch.Tensor          # bf16 [rows, hidden]
    scale: torch.Tensor      # bf16 [hidden]
    shift: torch.Tensor      # bf16 [hidden]
    input_scale: float       # fp32 static FP8 scale
    eps: float


def norm_modulate_inputs(rows: int, hidden: int = 3072, seed: int = 0,
                         input_scale: float = 0.0625, eps: float = 1e-6) -> NormModulateInputs:
    """x ~ N(0,1); scale, shift ~ N(0, 0.1) per column."""
    g = _gen(seed)
    x = _normal_bf16(g, (rows, hidden))
    scale = _normal_bf16(g, (hidden,), std=0.1)
    shift = _normal_bf16(g, (hidden,), std=0.1)
    return NormModulateInputs(x, scale, shift, float(np.float32(input_scale)), eps)


@dataclass
class ScaleResidualInputs:
    x: torch.Tensor          # bf16 [rows, hidden]
    residual: torch.Tensor   # bf16 [rows, hidden]
    bias: torch.Tensor | None  # bf16 [hidden]
    gate: torch.Tensor       # bf16 [hidden]
    scale: torch.Tensor      # bf16 [hidden]
    shift: torch.Tensor      # bf16 [hidden]
    input_scale: float
    eps: float


def scale_residual_inputs(rows: int, hidden: int = 3072, seed: int = 0,
                          input_scale: float = 0.0625, eps: float = 1e-6,
                          with_bias: bool = True) -> ScaleResidualInputs:
    """x, residual ~ N(0,1); bias ~ N(0, 0.02); gate ~ N(1, 0.1);
    scale, shift ~ N(0, 0.1)."""
    g = _gen(seed)
    x = _normal_bf16(g, (rows, hidden))
    residual = _normal_bf16(g, (rows, hidden))
    bias = _normal_bf16(g, (hidden,), std=0.02)
    gate = _normal_bf16(g, (hidden,), mean=1.0, std=0.1)
    scale = _normal_bf16(g, (hidden,), std=0.1)
    shift = _normal_bf16(g, (hidden,), std=0.1)
    return ScaleResidualInputs(x, residual, bias if with_bias else None, gate, scale,
                               shift, float(np.float32(input_scale)), eps)


def rope_tables(positions: np.ndarray, head_dim: int = 128, theta: float = 10000.0):
    """fp32 cos/sin tables [len(positions), head_dim/2]: angle = p * theta^(-2i/D),
    evaluated in binary64 and rounded to binary32 (the cache is an input)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * i / head_dim)
    ang = positions.astype(np.float64)[:, None] * inv_freq[None, :]
    return (np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32))


@dataclass
class QkvInputs:
    img_qkv: torch.Tensor    # bf16 [img_rows, 3 * heads * head_dim] (packed GEMM output)
    txt_qkv: torch.Tensor    # bf16 [txt_rows, 3 * heads * head_dim]
    img_q_w: torch.Tensor    # bf16 [head_dim]
    img_k_w: torch.Tensor
    txt_q_w: torch.Tensor
    txt_k_w: torch.Tensor
    img_cos: np.ndarray      # fp32 [img_rows, head_dim/2]
    img_sin: np.ndarray
    txt_cos: np.ndarray      # fp32 [txt_rows, head_dim/2]
    txt_sin: np.ndarray
    heads: int
    head_dim: int
    img_eps: float
    txt_eps: float

    @property
    def width(self) -> int:
        return self.heads * self.head_dim

    def views(self, which: str):
        """(q, k, v) column views of the packed buffer for 'img' or 'txt'."""
        t = self.img_qkv if which == "img" else self.txt_qkv
        w = self.width
        return t[:, 0:w], t[:, w:2 * w], t[:, 2 * w:3 * w]


def qkv_inputs(img_rows: int = 4096, txt_rows: int = 512, heads: int = 24,
               head_dim: int = 128, seed: int = 0, img_eps: float = 1e-6,
               txt_eps: float = 1e-6, theta: float = 10000.0) -> QkvInputs:
    """Packed QKV ~ N(0,1); four RMSNorm weights ~ N(1, 0.05); RoPE positions
    are joint indices: text 0..txt_rows-1, image txt_rows..txt_rows+img_rows-1."""
    g = _gen(seed)
    w = heads * head_dim
    img = _normal_bf16(g, (img_rows, 3 * w))
    txt = _normal_bf16(g, (txt_rows, 3 * w))
    ws = [_normal_bf16(g, (head_dim,), mean=1.0, std=0.05) for _ in range(4)]
    txt_cos, txt_sin = rope_tables(np.arange(txt_rows), head_dim, theta)
    img_cos, img_sin = rope_tables(np.arange(txt_rows, txt_rows + img_rows), head_dim, theta)
    return QkvInputs(img, txt, ws[0], ws[1], ws[2], ws[3], img_cos, img_sin,
                     txt_cos, txt_sin, heads, head_dim, img_eps, txt_eps)


@dataclass
class BiasMulAddInputs:
    x: torch.Tensor
    bias: torch.Tensor | None
    gate: torch.Tensor
    residual: torch.Tensor


def bias_mul_add_inputs(rows: int = 4608, hidden: int = 3072, seed: int = 0,
                        with_bias: bool = True) -> BiasMulAddInputs:
    """x, residual ~ N(0,1); bias ~ N(0, 0.02); gate ~ N(0, 0.5)."""
    g = _gen(seed)
    x = _normal_bf16(g, (rows, hidden))
    residual = _normal_bf16(g, (rows, hidden))
    bias = _normal_bf16(g, (hidden,), std=0.02)
    gate = _normal_bf16(g, (hidden,), std=0.5)
    return BiasMulAddInputs(x, bias if with_bias else None, gate, residual)


@dataclass
class TokenCatInputs:
    attn: torch.Tensor       # bf16 [rows, a_cols]
    mlp: torch.Tensor        # bf16 [rows, b_cols]
    fp8_scale: float         # static FP8 input scale
    fp4_g: float             # global fp32 inverse scale for FP4


def fp4_global_scale(*tensors: torch.Tensor) -> float:
    """Per-tensor calibration of the global FP4 inverse scale:
    g = RN32(448 * 6 / amax) over all given tensors (1.0 if all zero)."""
    amax = 0.0
    for t in tensors:
        if t.numel():
            amax = max(amax, float(t.float().abs().max()))
    if amax == 0.0:
        return 1.0
    return float(np.float32(np.float32(448.0 * 6.0) / np.float32(amax)))


def token_cat_inputs(rows: int = 4608, a_cols: int = 6144, b_cols: int = 18432,
                     seed: int = 0, fp8_scale: float = 0.05) -> TokenCatInputs:
    """attention and MLP branch outputs ~ N(0,1)."""
    g = _gen(seed)
    a = _normal_bf16(g, (rows, a_cols))
    b = _normal_bf16(g, (rows, b_cols))
    return TokenCatInputs(a, b, float(np.float32(fp8_scale)), fp4_global_scale(a, b))
