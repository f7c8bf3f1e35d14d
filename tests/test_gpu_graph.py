"""The training step (quantizers, forward, backward) captured once in a HIP graph through
torch.cuda.CUDAGraph, the library launching on the capture stream, and replayed: every replay gives
the eager step's outputs bit for bit (every kernel of the step is deterministic and none records a
memset), with eager steps, output clobbering and synchronizations between the replays."""
import math

import numpy as np
import pytest
import torch

import precision_mxfp8_block_amd as mx
import synth
from mx_cases import cu_dev, say, to_dev_bf16

pytestmark = pytest.mark.gpu


class Step:
    def __init__(self, lens, H=2, seed=61):
        self.lens = lens
        self.cu = synth.cu_seqlens(lens)
        T, C = int(self.cu[-1]), H * 128
        self.T, self.C, self.H = T, C, H
        self.cu_d = cu_dev(self.cu)
        self.x = {n: to_dev_bf16(synth.normal_bf16(seed, st, (T, C)))
                  for n, st in (("q", synth.STREAM_Q), ("k", synth.STREAM_K), ("v", synth.STREAM_V),
                                ("do", synth.STREAM_DO))}
        self.jag = any(L % 128 for L in lens)
        nb = int(np.sum((np.array(lens) + 31) // 32))
        P = mx.mxfa_padded_token_rows(self.cu)
        u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device="cuda")
        self.pay = {n: u8(T, C) for n in ("q", "k", "vc", "vr", "do")}
        self.sc = {"q": u8(nb, C // 32), "k": u8(nb, C // 32), "do": u8(nb, C // 32), "vc": u8(nb, C),
                   "vr": u8(T, C // 32)}
        self.pad = {n: (u8(P // 32, C // 32) if n in ("q", "k", "do") else u8(P // 32, C) if n == "vc" else
                        u8(P, C // 32)) if self.jag else self.sc[n] for n in self.sc}
        c = float(np.float32(1 / math.sqrt(128)))
        op = lambda n, mode: mx.MxOperand(self.pay[n], self.pad[n], mode)
        self.args = mx.AttnArgs(op("q", mx.SQ32), op("k", mx.SQ32), op("vc", mx.COL32), self.cu_d, self.cu_d,
                                len(lens), max(lens), max(lens), T, T, H, 128, c, False)
        self.vop, self.doop = op("vr", mx.ROW32), op("do", mx.SQ32)
        self.ws_bytes = mx.mxfa_bwd_workspace_size(self.args, 1)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")
        self.out = {"o": torch.empty((T, C), dtype=torch.bfloat16, device="cuda"),
                    "lse": torch.empty((H, T), dtype=torch.float32, device="cuda")}
        for n in ("dq", "dk", "dv"):
            self.out[n] = torch.empty((T, C), dtype=torch.bfloat16, device="cuda")

    def run(self, s):
        """One step, every launch on stream s."""
        L, B, T, C = max(self.lens), len(self.lens), self.T, self.C
        for n in ("q", "k", "do"):
            mx.mxfa_quantize(self.x[n], C, T, C, self.cu_d, B, L, mx.SQ32, self.pay[n], self.sc[n], None, s)
        mx.mxfa_quantize_col32_row32(self.x["v"], C, T, C, self.cu_d, B, L, self.pay["vc"], self.sc["vc"],
                                     self.pay["vr"], self.sc["vr"], s)
        if self.jag:
            for n, mode in (("q", mx.SQ32), ("k", mx.SQ32), ("do", mx.SQ32), ("vc", mx.COL32), ("vr", mx.ROW32)):
                mx.mxfa_varlen_scale_scatter(self.sc[n], self.cu_d, B, L, C, mode, self.pad[n], self.pad[n].shape[0], s)
        mx.mxfa_fwd(self.args, self.out["o"], self.out["lse"], s)
        mx.mxfa_bwd(self.args, self.vop, self.doop, self.out["o"], self.x["do"], self.out["lse"], 1, 1.0, self.ws,
                    self.ws_bytes, self.out["dq"], self.out["dk"], self.out["dv"], s)

    def clobber(self):
        for t in self.out.values():
            t.fill_(float("nan"))

    def snapshot(self):
        return {n: t.detach().cpu().clone() for n, t in self.out.items()}


def _same(a, b, label):
    for n in a:
        x, y = a[n].view(torch.int16 if a[n].dtype == torch.bfloat16 else torch.int32), \
            b[n].view(torch.int16 if b[n].dtype == torch.bfloat16 else torch.int32)
        assert torch.equal(x, y), f"{label}: {n} differs from the eager step"


@pytest.mark.parametrize("lens", [[512, 512], [300, 1000, 77]], ids=["uniform", "jagged"])
def test_training_step_graph_replay(lens):
    say(f"training step in a HIP graph, lengths {lens}")
    st = Step(lens)
    st.clobber()
    st.run(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = st.snapshot()
    assert all(torch.isfinite(t.float()).all() for t in ref.values() if t.dtype != torch.float32)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.run(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for r in range(3):
        st.clobber()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(st.snapshot(), ref, f"replay {r}")
        st.clobber()
        st.run(torch.cuda.current_stream())  # eager work between the replays
        torch.cuda.synchronize()
        _same(st.snapshot(), ref, f"eager step after replay {r}")
    say("  3 replays equal the eager step bit for bit")
