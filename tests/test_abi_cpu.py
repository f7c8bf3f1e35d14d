"""CPU tests of the boundary: the library loads and exports every entry point the header declares,
every argument error is reported before anything is enqueued (no GPU needed: the calls below fail
validation, so no HIP call is made), and host-only helpers compute what the header states."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import precision_mxfp8_block_amd as mx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxfa.h")

OK, INVALID, UNSUPPORTED = 0, 1, 2
P = 0x100000  # an aligned, never dereferenced stand-in pointer


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mxfa_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_abi():
    names = _declared_functions()
    for n in ["mxfa_quantize", "mxfa_quantize_col32_row32", "mxfa_quantize_e2m1", "mxfa_quantize_e2m3", "mxfa_fwd", "mxfa_fwd_p_scale", "mxfa_fwd_mx_out", "mxfa_bwd", "mxfa_bwd_mx_out",
              "mxfa_varlen_scale_scatter",
              "mxfa_rmsnorm_quantize",
              "mxfa_linear_quantize", "mxfa_linear_bwd_data", "mxfa_linear_bwd_weight",
              "mxfa_linear_bwd_weight_workspace_size", "mxfa_rmsnorm_bwd", "mxfa_rmsnorm_bwd_workspace_size",
              "mxfa_bwd_workspace_size", "mxfa_status_string", "mxfa_last_error_message"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(mx.library_path())
    for n in _declared_functions():
        assert hasattr(lib, n), n


def _lib():
    return mx._load()


def _last():
    return mx.mxfa_last_error_message()


@pytest.mark.parametrize("kw,expect", [
    (dict(mode=7), INVALID),
    (dict(C=48), INVALID),
    (dict(ld_x=100), INVALID),          # ld_x < C
    (dict(ld_x=132), INVALID),          # not a multiple of 8
    (dict(x=0), INVALID),
    (dict(x=P + 8), INVALID),           # misaligned
    (dict(T=-1), INVALID),
    (dict(scale_t=P), INVALID),         # scale_t only for SQ32 (mode ROW32 here)
    (dict(mode=2, cu=0), INVALID),      # jagged modes need cu_seqlens
    (dict(mode=2, nseq=0), INVALID),
    (dict(mode=1, max_seqlen=10 ** 6), INVALID),  # > T
])
def test_quantize_argument_errors(kw, expect):
    a = dict(x=P, ld_x=128, T=256, C=128, cu=P, nseq=1, max_seqlen=256, mode=0, data=P, scale=P, scale_t=0)
    a.update(kw)
    st = _lib().mxfa_quantize(a["x"], a["ld_x"], a["T"], a["C"], a["cu"], a["nseq"], a["max_seqlen"], a["mode"],
                              a["data"], a["scale"], a["scale_t"], 0)
    assert st == expect
    assert _last() != ""
    assert mx.mxfa_status_string(st) == {INVALID: "MXFA_ERR_INVALID", UNSUPPORTED: "MXFA_ERR_UNSUPPORTED"}[expect]


def _args(**kw):
    a = dict(q=(P, P, 2), k=(P, P, 2), v=(P, P, 1), cu_q=P, cu_k=P, nseq=1, max_q=256, max_k=256, total_q=256,
             total_k=256, H=1, D=128, scale=0.088, causal=0)
    a.update(kw)
    return mx._AttnArgs(mx._Mx(*a["q"]), mx._Mx(*a["k"]), mx._Mx(*a["v"]), a["cu_q"], a["cu_k"], a["nseq"],
                        a["max_q"], a["max_k"], a["total_q"], a["total_k"], a["H"], a["D"], a["scale"], a["causal"])


@pytest.mark.parametrize("kw,expect", [
    (dict(D=64), UNSUPPORTED),
    (dict(H=0), INVALID),
    (dict(H=65536), INVALID),           # a grid dimension of the backward's preprocess
    (dict(nseq=0), INVALID),
    (dict(max_q=300), INVALID),         # > total_q
    (dict(cu_q=0), INVALID),
    (dict(q=(P, P, 1)), INVALID),       # q must be ROW32 or SQ32
    (dict(v=(P, P, 0)), INVALID),       # v must be COL32 or SQ32
    (dict(k=(0, P, 2)), INVALID),
    (dict(k=(P + 4, P, 2)), INVALID),
    (dict(scale=float("inf")), INVALID),
    # element formats: MXFP4 only for q and k together, ROW32, with an E4M3 v
    (dict(q=(P, P, 0, 1), k=(P, P, 0, 0)), INVALID),      # q and k in different formats
    (dict(q=(P, P, 2, 1), k=(P, P, 2, 1)), UNSUPPORTED),  # MXFP4 in SQ32
    (dict(q=(P, P, 0, 1), k=(P, P, 0, 1), v=(P, P, 1, 1)), UNSUPPORTED),  # MXFP4 v
    (dict(q=(P, P, 0, 3), k=(P, P, 0, 3)), INVALID),      # not an element format
    (dict(q=(P, P, 0, 2), k=(P, P, 0, 1)), INVALID),      # MXFP6 q with MXFP4 k
    (dict(q=(P, P, 2, 2), k=(P, P, 2, 2)), UNSUPPORTED),  # MXFP6 in SQ32
])
def test_fwd_argument_errors(kw, expect):
    a = _args(**kw)
    st = _lib().mxfa_fwd(ctypes.byref(a), P, P, 0)
    assert st == expect, _last()
    assert _last() != ""


def test_bwd_rejects_mxfp4_operands():
    a = _args(q=(P, P, 0, 1), k=(P, P, 0, 1))
    need = mx.mxfa_bwd_workspace_size(a, 0)
    st = _lib().mxfa_bwd(ctypes.byref(a), mx._Mx(P, P, 0), mx._Mx(P, P, 2), P, P, P, 0, 1.0, P, need, P, P, P, 0)
    assert st == UNSUPPORTED and "E4M3" in _last()
    a = _args()
    st = _lib().mxfa_bwd(ctypes.byref(a), mx._Mx(P, P, 0, 1), mx._Mx(P, P, 2), P, P, P, 0, 1.0, P, need, P, P, P, 0)
    assert st == UNSUPPORTED


@pytest.mark.parametrize("kw,expect", [
    (dict(C=48), INVALID),
    (dict(ld_x=100), INVALID),
    (dict(ld_x=132), INVALID),
    (dict(x=0), INVALID),
    (dict(data=P + 8), INVALID),
    (dict(T=-1), INVALID),
])
def test_quantize_e2m1_argument_errors(kw, expect):
    a = dict(x=P, ld_x=128, T=256, C=128, data=P, scale=P)
    a.update(kw)
    for fn in (_lib().mxfa_quantize_e2m1, _lib().mxfa_quantize_e2m3):
        st = fn(a["x"], a["ld_x"], a["T"], a["C"], a["data"], a["scale"], 0)
        assert st == expect and _last() != ""


def test_quantize_e2m3_needs_block_pairs():
    # the MXFP6 payload stores blocks in pairs: C must be a multiple of 64 (96 is fine for MXFP4)
    assert _lib().mxfa_quantize_e2m3(P, 96, 256, 96, P, P, 0) == INVALID and "64" in _last()


def test_fwd_null_outputs():
    a = _args()
    assert _lib().mxfa_fwd(ctypes.byref(a), 0, P, 0) == INVALID
    assert _lib().mxfa_fwd(None, P, P, 0) == INVALID


@pytest.mark.parametrize("p_scale", [-1, 2, 7])
def test_fwd_p_scale_rejects_unknown_mode(p_scale):
    a = _args()
    assert _lib().mxfa_fwd_p_scale(ctypes.byref(a), p_scale, P, P, 0) == INVALID
    assert "p_scale" in _last()


@pytest.mark.parametrize("o,o_data,o_scale,lse", [
    (0, 0, 0, P),         # neither output
    (0, P, 0, P),         # MX payload without its scales
    (P, P + 2, P, P),     # payload not 4-byte aligned
    (0, P, P + 1, P),     # scales not 4-byte aligned
    (P + 8, 0, 0, P),     # bf16 O not 16-byte aligned
    (P, P, P, 0),         # no LSE
])
def test_fwd_mx_out_argument_errors(o, o_data, o_scale, lse):
    a = _args()
    assert _lib().mxfa_fwd_mx_out(ctypes.byref(a), mx.P_STATIC, o, o_data, o_scale, lse, 0) == INVALID
    assert _last() != ""


@pytest.mark.parametrize("kw", [dict(H=0), dict(v=(P, P, 0)), dict(scale=float("inf"))])
def test_fwd_p_scale_checks_the_problem_like_fwd(kw):
    a = _args(**kw)
    for mode in (mx.P_STATIC, mx.P_BLOCK_DYNAMIC):
        assert _lib().mxfa_fwd_p_scale(ctypes.byref(a), mode, P, P, 0) == INVALID


@pytest.mark.parametrize("kw,expect", [
    (dict(args=dict(q=(P, P, 0))), INVALID),   # backward needs SQ32 q and k
    (dict(vd_mode=1), INVALID),                # v_d must be along D
    (dict(do_mode=0), INVALID),                # dO must be SQ32
    (dict(dq_mode=1, sigma=3.0), INVALID),     # sigma not a power of two
    (dict(dq_mode=1, sigma=0.0), INVALID),
    (dict(dq_mode=5), INVALID),
    (dict(ws_bytes=16), INVALID),              # workspace too small
    (dict(ws=P + 64), INVALID),                # workspace not 256-aligned
])
def test_bwd_argument_errors(kw, expect):
    a = _args(**kw.get("args", {}))
    need = mx.mxfa_bwd_workspace_size(a, 0)
    st = _lib().mxfa_bwd(ctypes.byref(a), mx._Mx(P, P, kw.get("vd_mode", 0)), mx._Mx(P, P, kw.get("do_mode", 2)), P, P,
                         P, kw.get("dq_mode", 0), kw.get("sigma", 1.0), kw.get("ws", P), kw.get("ws_bytes", need), P,
                         P, P, 0)
    assert st == expect, _last()


@pytest.mark.parametrize("bf16,mxp", [
    ((0, 0, 0), None),                      # no gradient output at all
    ((P, 0, 0), None),                      # bf16 gradients only partly given
    ((0, 0, 0), (P, P, P, 0, P, P)),        # an MXFP8 scale pointer missing
    ((0, 0, 0), (P, P, P + 8, P, P, P)),    # an MXFP8 payload not 16-byte aligned
    ((P, P, P + 8, ), (P, P, P, P, P, P)),  # bf16 dv misaligned
])
def test_bwd_mx_out_argument_errors(bf16, mxp):
    a = _args()
    need = mx.mxfa_bwd_workspace_size(a, 0)
    bf16 = tuple(bf16) + (0,) * (3 - len(bf16))
    g = ctypes.byref(mx._GradMx(*mxp)) if mxp is not None else None
    st = _lib().mxfa_bwd_mx_out(ctypes.byref(a), mx._Mx(P, P, 0), mx._Mx(P, P, 2), P, P, P, 0, 1.0, P, need, *bf16, g, 0)
    assert st == INVALID, _last()
    assert _last() != ""


def test_scatter_and_rmsnorm_argument_errors():
    lib = _lib()
    assert lib.mxfa_varlen_scale_scatter(P, P, 1, 256, 100, 0, P, 256, 0) == INVALID  # C % 32
    assert lib.mxfa_varlen_scale_scatter(P, P, 1, 256, 128, 0, P, 100, 0) == INVALID  # padded_rows too small
    assert lib.mxfa_varlen_scale_scatter(0, P, 1, 256, 128, 0, P, 256, 0) == INVALID
    assert lib.mxfa_rmsnorm_quantize(P, 1024, 64, 1024, P, -1.0, P, 1, 64, P, P, 0, 0) == INVALID  # eps < 0
    assert lib.mxfa_rmsnorm_quantize(P, 1024, 64, 1024, 0, 1e-6, P, 1, 64, P, P, 0, 0) == INVALID  # gamma NULL
    assert lib.mxfa_rmsnorm_quantize(P, 1024, 64, 1000, P, 1e-6, P, 1, 64, P, P, 0, 0) == INVALID  # C % 32


def test_workspace_size_and_padded_rows():
    # H * nseq * ceil(max_q/128) * ceil(max_k/128) dS tiles of 16 KB, their 16-byte code blocks, then two
    # fp32 [H][Tq] vectors; each region rounded up to 256 bytes
    a = _args(nseq=3, max_q=300, max_k=129, total_q=1000, total_k=1000, H=2)
    tiles = 2 * 3 * 3 * 2
    al = lambda x: (x + 255) // 256 * 256
    expect = al(tiles * 16384) + al(tiles * 16) + 2 * al(1000 * 2 * 4)
    assert mx.mxfa_bwd_workspace_size(a, 0) == expect
    assert mx.mxfa_bwd_workspace_size(a, 1) == expect
    assert mx.mxfa_bwd_workspace_size(_args(H=0), 0) == 0
    assert mx.mxfa_padded_token_rows(np.array([0, 1, 129, 129, 385], np.int32)) == 128 + 128 + 0 + 256


def test_device_code_has_no_packed_fp32_instructions():
    """Every kernel file compiled for gfx950 contains no packed-FP32 VALU instruction."""
    csrc = os.path.join(ROOT, "precision_mxfp8_block_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if not f.endswith(".hip"):
            continue
        r = subprocess.run(["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-S",
                            "--cuda-device-only", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                            "-I", os.path.join(ROOT, "include"), "-I", csrc, os.path.join(csrc, f), "-o", "-"],
                           capture_output=True, text=True, check=True)
        bad = [l for l in r.stdout.splitlines() if re.search(r"\bv_pk_(add|mul|fma)_f32\b", l)]
        assert not bad, (f, bad[:3])


@pytest.mark.parametrize("kw,expect", [
    (dict(C_in=96), INVALID),            # C_in must be a multiple of 128
    (dict(C_out=160), INVALID),          # C_out must be a multiple of 128
    (dict(x=(P, P, 1)), INVALID),        # x must be SQ32 or ROW32
    (dict(w=(P, P, 2)), INVALID),        # w must be ROW32
    (dict(x=(0, P, 2)), INVALID),
    (dict(w=(P, P + 4, 0)), INVALID),    # misaligned scale
    (dict(data=0), INVALID),
    (dict(nseq=0), INVALID),
    (dict(max_seqlen=300), INVALID),     # > T
    (dict(T=-1), INVALID),
])
def test_linear_quantize_argument_errors(kw, expect):
    a = dict(x=(P, P, 2), w=(P, P, 0), T=256, C_in=1024, C_out=1024, cu=P, nseq=1, max_seqlen=256, data=P, scale=P,
             scale_t=0)
    a.update(kw)
    st = _lib().mxfa_linear_quantize(mx._Mx(*a["x"]), mx._Mx(*a["w"]), a["T"], a["C_in"], a["C_out"], a["cu"],
                                     a["nseq"], a["max_seqlen"], a["data"], a["scale"], a["scale_t"], 0)
    assert st == expect, _last()
    assert _last() != ""


def test_bwd_no_alloc_argument_errors():
    """The allocation-free backward rejects, before any HIP call, missing outputs and problems whose
    workspace exceeds its fixed array (B=4, H=16, N=4096 needs about 1 GB); the limit is 64 MiB."""
    lib = _lib()
    assert mx.mxfa_bwd_no_alloc_max_workspace() == 64 << 20
    big = _args(nseq=4, max_q=4096, max_k=4096, total_q=16384, total_k=16384, H=16)
    assert mx.mxfa_bwd_workspace_size(big, 1) > mx.mxfa_bwd_no_alloc_max_workspace()
    st = lib.mxfa_bwd_no_alloc(ctypes.byref(big), mx._Mx(P, P, 0), mx._Mx(P, P, 2), P, P, P, 1, 1.0, P, P, P, 0)
    assert st == INVALID and "mxfa_bwd_no_alloc" in _last() and "workspace" in _last()
    small = _args()
    assert lib.mxfa_bwd_no_alloc(ctypes.byref(small), mx._Mx(P, P, 0), mx._Mx(P, P, 2), P, P, P, 1, 1.0, 0, P, P,
                                 0) == INVALID
    assert lib.mxfa_bwd_no_alloc(ctypes.byref(small), mx._Mx(P, P, 0), mx._Mx(P, P, 1), P, P, P, 1, 1.0, P, P, P,
                                 0) == INVALID  # dO must be SQ32


@pytest.mark.parametrize("kw,expect", [
    (dict(C_out=96), INVALID),           # C_out (the contraction) must be a multiple of 128
    (dict(C_in=160), INVALID),           # C_in must be a multiple of 128
    (dict(dy=(P, P, 1)), INVALID),       # dy must be SQ32 or ROW32
    (dict(wt=(P, P, 2)), INVALID),       # W^T must be ROW32 (scales along C_out)
    (dict(dy=(0, P, 2)), INVALID),
    (dict(wt=(P, P + 4, 0)), INVALID),   # misaligned scale
    (dict(dx=P + 2), INVALID),           # misaligned output
    (dict(dx=0), INVALID),
    (dict(nseq=0), INVALID),
    (dict(T=-1), INVALID),
    (dict(accumulate=2), INVALID),
])
def test_linear_bwd_data_argument_errors(kw, expect):
    a = dict(dy=(P, P, 2), wt=(P, P, 0), T=256, C_out=1024, C_in=1024, cu=P, nseq=1, max_seqlen=256, accumulate=0,
             dx=P)
    a.update(kw)
    st = _lib().mxfa_linear_bwd_data(mx._Mx(*a["dy"]), mx._Mx(*a["wt"]), a["T"], a["C_out"], a["C_in"], a["cu"],
                                     a["nseq"], a["max_seqlen"], a["accumulate"], a["dx"], 0)
    assert st == expect, _last()
    assert "mxfa_linear_bwd_data" in _last()


@pytest.mark.parametrize("kw,expect", [
    (dict(C_out=96), INVALID),
    (dict(C_in=160), INVALID),
    (dict(T=1 << 23), UNSUPPORTED),      # T x C reaches 2^32 bytes (32-bit load offsets)
    (dict(dy=0), INVALID),
    (dict(x_st=0), INVALID),
    (dict(dw=P + 4), INVALID),           # misaligned
    (dict(workspace=0), INVALID),
    (dict(workspace_bytes=16), INVALID),  # too small
    (dict(max_seqlen=300), INVALID),
])
def test_linear_bwd_weight_argument_errors(kw, expect):
    a = dict(dy=P, dy_st=P, x=P, x_st=P, T=256, C_out=1024, C_in=1024, cu=P, nseq=1, max_seqlen=256, workspace=P,
             workspace_bytes=1 << 40, dw=P)
    a.update(kw)
    st = _lib().mxfa_linear_bwd_weight(a["dy"], a["dy_st"], a["x"], a["x_st"], a["T"], a["C_out"], a["C_in"], a["cu"],
                                       a["nseq"], a["max_seqlen"], a["workspace"], a["workspace_bytes"], a["dw"], 0)
    assert st == expect, _last()
    assert "mxfa_linear_bwd_weight" in _last()


def test_linear_bwd_weight_workspace_size():
    """Block table (one int2 per token block, bounded by T/32 + nseq) plus one FP32 partial dW per token
    chunk; at least one partial, growing with T."""
    small = mx.mxfa_linear_bwd_weight_workspace_size(256, 1, 1024, 1024)
    big = mx.mxfa_linear_bwd_weight_workspace_size(75659, 64, 1024, 1024)
    assert small >= 1024 * 1024 * 4 and big > small
    assert big % 4 == 0
    assert mx.mxfa_linear_bwd_weight_workspace_size(-1, 1, 1024, 1024) == 0


@pytest.mark.parametrize("kw,expect", [
    (dict(C=48), UNSUPPORTED),           # multiple of 32
    (dict(C=4096), UNSUPPORTED),         # above 2048
    (dict(ld_x=100), INVALID),
    (dict(x=P + 8), INVALID),
    (dict(dgamma=P + 4), INVALID),       # float4 stores
    (dict(eps=float("nan")), INVALID),
    (dict(workspace_bytes=64), INVALID),
    (dict(dy=0), INVALID),
    (dict(T=-1), INVALID),
])
def test_rmsnorm_bwd_argument_errors(kw, expect):
    a = dict(x=P, ld_x=1024, T=128, C=1024, gamma=P, eps=1e-6, dy=P, workspace=P, workspace_bytes=1 << 40, dx=P,
             dgamma=P)
    a.update(kw)
    st = _lib().mxfa_rmsnorm_bwd(a["x"], a["ld_x"], a["T"], a["C"], a["gamma"], a["eps"], a["dy"], a["workspace"],
                                 a["workspace_bytes"], a["dx"], a["dgamma"], 0)
    assert st == expect, _last()
    assert "mxfa_rmsnorm_bwd" in _last()


@pytest.mark.parametrize("kw,expect", [
    (dict(C=48), INVALID),
    (dict(ld_x=100), INVALID),
    (dict(ld_x=132), INVALID),
    (dict(x=0), INVALID),
    (dict(cu=0), INVALID),              # the COL32 blocks follow the sequences
    (dict(nseq=0), INVALID),
    (dict(max_seqlen=300), INVALID),    # > T
    (dict(dc=P + 8), INVALID),
    (dict(sc=0), INVALID),
    (dict(dr=P + 4), INVALID),
    (dict(sr=0), INVALID),
    (dict(T=-1), INVALID),
])
def test_quantize_col32_row32_argument_errors(kw, expect):
    a = dict(x=P, ld_x=128, T=256, C=128, cu=P, nseq=2, max_seqlen=128, dc=P, sc=P, dr=P, sr=P)
    a.update(kw)
    st = _lib().mxfa_quantize_col32_row32(a["x"], a["ld_x"], a["T"], a["C"], a["cu"], a["nseq"], a["max_seqlen"],
                                          a["dc"], a["sc"], a["dr"], a["sr"], 0)
    assert st == expect and "mxfa_quantize_col32_row32" in _last()


@pytest.mark.parametrize("first,n,variant,sc", [(0, 6, 0, 1.0), (0, 8, 3, 1.0), (0, 8, -1, 1.0), (0, 8, 1, 3.0),
                                                (0, 8, 1, 2.0 ** 120), (0, 8, 1, 2.0 ** -127), (0, -4, 0, 1.0),
                                                (0, (1 << 32) + 4, 0, 1.0)])
def test_e4m3_pack_patterns_argument_errors(first, n, variant, sc):
    lib = _lib()
    assert lib.mxfa_e4m3_pack_patterns(first, n, variant, sc, P, None) == INVALID
    assert "mxfa_e4m3_pack_patterns" in _last()


def test_e4m3_pack_patterns_pointer_errors():
    lib = _lib()
    assert lib.mxfa_e4m3_pack_patterns(0, 8, 0, 1.0, None, None) == INVALID
    assert lib.mxfa_e4m3_pack_patterns(0, 8, 0, 1.0, P + 2, None) == INVALID
    assert lib.mxfa_e4m3_pack_patterns(0, 0, 0, 1.0, None, None) == OK  # nothing to write, no launch
