"""mxfa_bwd_no_alloc (the backward with the library's fixed per-GPU workspace array) against mxfa_bwd
with a caller-owned workspace, through the C ABI.

Both run the same kernels on the same inputs and the backward is deterministic (the dQ reduction
runs over the KV tiles in a fixed order), so the outputs must be bit-identical. Two calls in a row,
the second on a smaller problem (the array keeps the first call's contents, which the second must
not depend on); outputs are prefilled with NaN so an element the kernels never write cannot pass.
A problem whose workspace exceeds the array is rejected before anything is enqueued.
"""
import numpy as np
import pytest
import torch

import precision_mxfp8_block_amd as mx
from mx_cases import AttnCase, gpu_quantize_padded, say, to_host_bf16_bits

pytestmark = pytest.mark.gpu


def _nan_like(t):
    return torch.full_like(t, float("nan"))


def _both(case, dq_mode, sigma):
    c = case
    gvd = gpu_quantize_padded(c.v_d, c.cu_k, c.cu_k_d, mx.ROW32)
    gdo = gpu_quantize_padded(c.do_d, c.cu_q, c.cu_q_d, mx.SQ32)
    vop, doop = mx.MxOperand(gvd[0], gvd[1], mx.ROW32), mx.MxOperand(gdo[0], gdo[1], mx.SQ32)
    ref = mx.bwd(c.args, vop, doop, c.o_dev, c.do_d, c.lse_dev, dq_mode, sigma)
    out = tuple(_nan_like(t) for t in ref)
    mx.mxfa_bwd_no_alloc(c.args, vop, doop, c.o_dev, c.do_d, c.lse_dev, dq_mode, sigma, *out)
    torch.cuda.synchronize()
    return [to_host_bf16_bits(t) for t in ref], [to_host_bf16_bits(t) for t in out]


@pytest.mark.parametrize("dq_mode,sigma", [(mx.DQ_FP16_STATIC, 1.0), (mx.DQ_FP32, 1.0)])
def test_no_alloc_matches_workspace_backward(dq_mode, sigma):
    need_big = None
    for label, seed, lens, H, causal in (("first", 31, [512, 300, 77], 2, False), ("second_smaller", 32, [200], 1, True)):
        say(f"no-alloc bwd {label} lens={lens} H={H} causal={causal} dq_mode={dq_mode}")
        c = AttnCase(seed, lens, None, H=H, causal=causal)
        c.run_gpu_fwd()
        need = mx.mxfa_bwd_workspace_size(c.args, dq_mode)
        assert need <= mx.mxfa_bwd_no_alloc_max_workspace()
        if need_big is not None:
            assert need < need_big  # the second problem is the smaller one
        need_big = need
        ref, got = _both(c, dq_mode, sigma)
        for name, a, b in zip(("dq", "dk", "dv"), ref, got):
            assert np.all(np.isfinite((b.astype(np.uint32) << 16).view(np.float32))), name
            np.testing.assert_array_equal(b, a, err_msg=name)


def test_no_alloc_rejects_problems_beyond_the_array():
    """B=4, H=16, N=4096 needs about 1 GB of workspace: rejected with MXFA_ERR_INVALID and a message
    naming the limit; nothing is enqueued (no tensor is even touched)."""
    say("no-alloc bwd: oversized problem rejected")
    P = 1 << 20
    op = mx.MxOperand(P, P, mx.SQ32)
    a = mx.AttnArgs(op, op, mx.MxOperand(P, P, mx.COL32), P, P, 4, 4096, 4096, 16384, 16384, 16, 128, 0.088, False)
    assert mx.mxfa_bwd_workspace_size(a, 1) > mx.mxfa_bwd_no_alloc_max_workspace()
    with pytest.raises(mx.MxfaError, match="mxfa_bwd_no_alloc.*workspace"):
        mx.mxfa_bwd_no_alloc(a, mx.MxOperand(P, P, mx.ROW32), op, P, P, P, mx.DQ_FP16_STATIC, 1.0, P, P, P)
