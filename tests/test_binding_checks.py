"""The allocating torch wrappers refuse mismatched tensors before any call
(CPU only). The C ABI takes raw pointers and cannot see sizes, so a wrong
broadcast vector, residual, branch or table size must be stopped here: each
case below raises ValueError naming the offending argument. With every shape
right, CPU tensors are refused too (all tensors must sit on one GPU), so no
case reaches the library.
"""
import numpy as np
import pytest
import torch

import quant_epilogues_amd as qe

H = 256
bf = torch.bfloat16


def z(*shape, dtype=bf):
    return torch.zeros(*shape, dtype=dtype)


S = torch.ones(1)  # fp32 scalar


def test_norm_modulate_checks():
    x = z(4, H)
    with pytest.raises(ValueError, match="scale"):
        qe.norm_modulate_fp8(x, z(H + 8), z(H), S)
    with pytest.raises(ValueError, match="shift"):
        qe.norm_modulate_fp8(x, z(H), z(H - 8), S)
    with pytest.raises(ValueError, match="input_scale"):
        qe.norm_modulate_fp8(x, z(H), z(H), torch.ones(2))
    with pytest.raises(ValueError, match="x must be a bf16"):
        qe.norm_modulate_fp8(x.float(), z(H), z(H), S)
    with pytest.raises(ValueError, match="contiguous"):
        qe.norm_modulate_fp8(z(H, 4).t(), z(4), z(4), S)
    with pytest.raises(ValueError, match="one GPU"):
        qe.norm_modulate_fp8(x, z(H), z(H), S)
    with pytest.raises(ValueError, match="global_scale"):
        qe.norm_modulate_fp4(x, z(H), z(H), None)
    with pytest.raises(ValueError, match="one GPU"):
        qe.norm_modulate_fp4(x, z(H), z(H), S)


@pytest.mark.parametrize("fn", ["fp8", "fp4"])
def test_scale_residual_checks(fn):
    f = qe.scale_residual_norm_modulate_fp8 if fn == "fp8" else qe.scale_residual_norm_modulate_fp4
    x = z(4, H)
    good = dict(x=x, bias=z(H), gate=z(H), residual=z(4, H), scale=z(H), shift=z(H))
    for name, bad in (("residual", z(3, H)), ("residual", z(4, H + 8)), ("gate", z(H // 2)),
                      ("bias", z(H + 16)), ("scale", z(2, H)), ("shift", z(1))):
        args = dict(good, **{name: bad})
        with pytest.raises(ValueError, match=name):
            f(args["x"], args["bias"], args["gate"], args["residual"], args["scale"],
              args["shift"], S)
    with pytest.raises(ValueError, match="one GPU"):
        f(x, None, z(H), z(4, H), z(H), z(H), S)


def test_bias_mul_add_checks():
    x = z(4, H)
    with pytest.raises(ValueError, match="residual"):
        qe.bias_mul_add(x, z(H), z(H), z(5, H))
    with pytest.raises(ValueError, match="gate"):
        qe.bias_mul_add(x, z(H), z(H - 8), z(4, H))
    with pytest.raises(ValueError, match="bias"):
        qe.bias_mul_add(x, z(2 * H), z(H), z(4, H))
    with pytest.raises(ValueError, match="one GPU"):
        qe.bias_mul_add(x, None, z(H), z(4, H))


def test_token_cat_checks():
    a = z(8, 64)
    with pytest.raises(ValueError, match="b must be"):
        qe.token_cat_quant(qe.DIT_QUANT_FP8_E4M3, a, z(7, 32), S)
    with pytest.raises(ValueError, match="a must be"):
        qe.token_cat_quant(qe.DIT_QUANT_FP8_E4M3, z(64), None, S)
    with pytest.raises(ValueError, match="scale"):
        qe.token_cat_quant(qe.DIT_QUANT_FP4_E2M1, a, z(8, 32), torch.ones(1, dtype=torch.float64))
    with pytest.raises(ValueError, match="one GPU"):
        qe.token_cat_quant(qe.DIT_QUANT_FP4_E2M1, a, z(8, 32), S)


def _qkv_args(img=6, txt=2, heads=2, d=128):
    w = heads * d
    img_p, txt_p = z(img, 3 * w), z(txt, 3 * w)
    tab = lambda n: torch.zeros(n, d // 2)
    return dict(img_q=img_p[:, :w], img_k=img_p[:, w:2 * w], img_v=img_p[:, 2 * w:],
                txt_q=txt_p[:, :w], txt_k=txt_p[:, w:2 * w], txt_v=txt_p[:, 2 * w:],
                img_q_w=z(d), img_k_w=z(d), txt_q_w=z(d), txt_k_w=z(d),
                img_cos=tab(img), img_sin=tab(img), txt_cos=tab(txt), txt_sin=tab(txt),
                heads=heads)


def test_qkv_checks():
    good = _qkv_args()
    cases = [
        ("img_q_w", z(64)), ("txt_k_w", z(128).float()),
        ("img_cos", torch.zeros(5, 64)),            # fewer rows than the image stream
        ("txt_sin", torch.zeros(2, 32)),            # not head_dim / 2 wide
        ("img_sin", torch.zeros(6, 64, dtype=torch.float64)),
        ("img_k", z(5, 256)),                       # another row count than img_q
        ("txt_v", z(2, 512)[:, :256]),              # another row stride than txt_q
        ("img_q", z(6, 255)),
    ]
    for name, bad in cases:
        with pytest.raises(ValueError, match=name):
            qe.qkv_epilogue(**dict(good, **{name: bad}))
    cache = torch.zeros(8, 128)  # [cos | sin] rows: tables with another row stride
    with pytest.raises(ValueError, match="one row stride"):
        qe.qkv_epilogue(**dict(good, img_cos=cache[2:, :64]))
    with pytest.raises(ValueError, match="one GPU"):
        qe.qkv_epilogue(**good)


def test_norm_dual_checks():
    img, txt = z(8, H), z(2, H)
    with pytest.raises(ValueError, match="txt_x must have hidden"):
        qe.norm_modulate_fp8_dual(img, z(H), z(H), S, z(2, H + 8), z(H), z(H), S)
    with pytest.raises(ValueError, match="txt_scale"):
        qe.norm_modulate_fp8_dual(img, z(H), z(H), S, txt, z(H - 8), z(H), S)
    with pytest.raises(ValueError, match="img_input_scale"):
        qe.norm_modulate_fp8_dual(img, z(H), z(H), None, txt, z(H), z(H), S)
    with pytest.raises(ValueError, match="one GPU"):
        qe.norm_modulate_fp8_dual(img, z(H), z(H), S, txt, z(H), z(H), S)
