"""GPU backward cases in which one quantization point of the method decides the gradients.

On N(0,1) inputs several plausible kernel mistakes move the gradients by less than the stated
tolerance. The structured inputs of synth.structured make each of them move some (32-token block,
head) of a gradient by more than ten times the tolerance (tests/test_oracle_mutations.py checks that
on the CPU by planting each mistake in the oracle), so these cases compare every such block, not only
the whole tensor:
  * Delta from the bf16 dO, not the quantized one (delta_sensitive: dO's N(0,1) entries quantize to
    zero next to 2^22-sized ones, and dS is carried by Delta alone);
  * dS quantized per 32 x 32 block (ds_block_range: dS spans ~2^18 between neighbouring key blocks
    of one query band);
  * the static P scale 2^-8 (p_subnormal_band: P of odd key blocks among E4M3 subnormals at 2^-8,
    below E4M3's range at scale 1);
  * binary16 round-to-nearest-even of the FP16 dQ accumulator with its static scale (dq_fp16_rounding:
    exact small values whose FP16 result is 1.5, against 1.0 when truncating and 1.375 in FP32).
"""
import numpy as np
import pytest
import torch

import precision_mxfp8_block_amd as mx
from mx_cases import (GRAD_REL_FRO, AttnCase, block_rel_errors, bf16_bits_to_f64, check_grads, check_o, say,
                      to_dev_bf16)
from synth import structured

pytestmark = pytest.mark.gpu

STRUCTURED = {
    "delta_sensitive": structured.delta_sensitive,
    "ds_block_range": structured.ds_block_range,
    "p_subnormal_band": structured.p_subnormal_band,
}


def check_blocks(g_bits, ref, lens_q, lens_k, H, label):
    for name, g, lens in zip(("dq", "dk", "dv"), g_bits, (lens_q, lens_k, lens_k)):
        errs = block_rel_errors(bf16_bits_to_f64(g), ref[name + "_f"], lens, H)
        worst = int(np.argmax(errs))
        say(f"  {label} {name}: {errs.size} blocks, max block rel_fro {errs[worst]:.3e} (block {worst}), "
            f"median {float(np.median(errs)):.3e}")
        assert errs[worst] <= GRAD_REL_FRO, (name, worst, errs[worst])


@pytest.mark.parametrize("dq_mode", [mx.DQ_FP16_STATIC, mx.DQ_FP32])
@pytest.mark.parametrize("name", list(STRUCTURED))
def test_structured_backward_blockwise(name, dq_mode):
    case = STRUCTURED[name]()
    lens, H = case["lens"], case["inputs"]["q"].shape[1] // 128
    say(f"structured bwd {name} lens={lens} H={H} dq_mode={dq_mode}")
    c = AttnCase(0, lens, None, H=H, softmax_scale=case["softmax_scale"], inputs=case["inputs"])
    o_gpu, lse_gpu = c.run_gpu_fwd()
    _, o32, lse = c.run_oracle_fwd()
    check_o(o_gpu, o32, lse_gpu, lse, name)
    g = c.run_gpu_bwd(dq_mode, 1.0)
    ref = c.run_oracle_bwd(dq_mode, 1.0)
    assert ref["overflow"] == 0
    check_grads(g, ref, name)
    check_blocks(g, ref, lens, lens, H, name)


@pytest.mark.parametrize("dq_mode,sigma,expect", [
    (mx.DQ_FP16_STATIC, 2.0 ** -23, 1.5),   # fp16(2^-23) + fp16(0.375 * 2^-23) = 2u + 1u (u = 2^-24), / sigma
    (mx.DQ_FP16_STATIC, 1.0, 1.375),        # 1 + 0.375 is exact in binary16
    (mx.DQ_FP32, 1.0, 1.375),
])
def test_dq_fp16_rounding_exact(dq_mode, sigma, expect):
    """Exact inputs (synth.structured.dq_fp16_rounding) with O = 0 and LSE = 0 given to the backward:
    every GPU gradient equals the oracle's bit for bit, and dQ[0, 1] is the hand-derived value. With
    sigma = 2^-23 the second partial, 0.375 * 2^-23 = 0.75 * 2^-24, is rounded to the nearest binary16
    subnormal 2^-24 (truncation would give 0 and dQ = 1.0)."""
    case = structured.dq_fp16_rounding()
    say(f"dq fp16 rounding dq_mode={dq_mode} sigma={sigma}")
    c = AttnCase(0, case["lens_q"], case["lens_k"], H=1, softmax_scale=case["softmax_scale"], inputs=case["inputs"])
    c.run_gpu_fwd()
    c.run_oracle_fwd()
    o0 = torch.zeros((1, 128), dtype=torch.bfloat16, device="cuda")
    lse0 = torch.zeros((1, 1), dtype=torch.float32, device="cuda")
    g = c.run_gpu_bwd(dq_mode, sigma, o=o0, lse=lse0)
    ref = c.run_oracle_bwd(dq_mode, sigma, o16=np.zeros((1, 128), np.uint16), lse=np.zeros((1, 1), np.float32))
    assert ref["dq_f"][0, 1] == np.float32(expect)
    for name, x in zip(("dq", "dk", "dv"), g):
        np.testing.assert_array_equal(x, ref[name], err_msg=name)
    assert bf16_bits_to_f64(g[0])[0, 1] == expect
