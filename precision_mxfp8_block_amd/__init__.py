"""MXFP8 block-scaled attention for AMD MI355X (gfx950): Python binding of libmxfa.so.

The functions named mxfa_* are the C ABI of include/mxfa.h, one to one: they only turn torch
tensors (device memory) and Python numbers into pointers and integers and raise MxfaError on a
non-OK status. Every step of the computation runs in the HIP kernels of libmxfa.so; there is no
fallback path. The allocate-and-call helpers at the end (quantize, scale_scatter, fwd, bwd,
rmsnorm_quantize, linear_quantize, linear_bwd_data, linear_bwd_weight, rmsnorm_bwd) size the output tensors
and workspaces with torch and call the same entry points.
"""
import ctypes
import os

import torch

__all__ = [
    "ROW32", "COL32", "SQ32", "DQ_FP32", "DQ_FP16_STATIC", "P_STATIC", "P_BLOCK_DYNAMIC", "MxfaError",
    "mxfa_quantize", "mxfa_varlen_scale_scatter", "mxfa_padded_token_rows", "mxfa_fwd", "mxfa_fwd_p_scale",
    "mxfa_fwd_mx_out", "mxfa_bwd", "mxfa_bwd_mx_out", "mxfa_bwd_no_alloc", "mxfa_bwd_no_alloc_max_workspace",
    "fwd_mx_out", "bwd_mx_out",
    "mxfa_bwd_workspace_size", "mxfa_rmsnorm_quantize", "mxfa_linear_quantize", "mxfa_status_string",
    "mxfa_last_error_message", "MxOperand", "AttnArgs", "quantize", "scale_scatter", "fwd", "bwd",
    "rmsnorm_quantize", "linear_quantize", "E4M3", "E2M1", "E2M3", "mxfa_quantize_e2m1", "mxfa_e4m3_pack_patterns",
    "quantize_e2m1", "mxfa_quantize_e2m3", "quantize_e2m3", "mxfa_quantize_col32_row32",
    "mxfa_linear_bwd_data", "mxfa_linear_bwd_weight", "mxfa_linear_bwd_weight_workspace_size", "mxfa_rmsnorm_bwd",
    "mxfa_rmsnorm_bwd_workspace_size", "linear_bwd_data", "linear_bwd_weight", "rmsnorm_bwd",
    "library_path",
]

ROW32, COL32, SQ32 = 0, 1, 2
DQ_FP32, DQ_FP16_STATIC = 0, 1
P_STATIC, P_BLOCK_DYNAMIC = 0, 1
E4M3, E2M1, E2M3 = 0, 1, 2  # element formats (mxfa_elem)

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmxfa.so")
_lib = None


class MxfaError(RuntimeError):
    pass


def library_path():
    return _LIB_PATH


class _Mx(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("mode", ctypes.c_int), ("elem", ctypes.c_int)]


class _GradMx(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("dq", "dq_scale", "dk", "dk_scale", "dv", "dv_scale", "dq_scale_t",
                                               "dk_scale_t", "dv_scale_t")]


class _AttnArgs(ctypes.Structure):
    _fields_ = [("q", _Mx), ("k", _Mx), ("v", _Mx),
                ("cu_seqlens_q", ctypes.c_void_p), ("cu_seqlens_k", ctypes.c_void_p),
                ("nseq", ctypes.c_int), ("max_seqlen_q", ctypes.c_int), ("max_seqlen_k", ctypes.c_int),
                ("total_q", ctypes.c_int64), ("total_k", ctypes.c_int64),
                ("num_heads", ctypes.c_int), ("head_dim", ctypes.c_int),
                ("softmax_scale", ctypes.c_float), ("causal", ctypes.c_int)]


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "(hipcc --offload-arch=gfx950); there is no fallback implementation")
    lib = ctypes.CDLL(_LIB_PATH)
    P, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    lib.mxfa_quantize.argtypes = [P, i64, i64, i32, P, i32, i32, i32, P, P, P, P]
    lib.mxfa_varlen_scale_scatter.argtypes = [P, P, i32, i32, i32, i32, P, i64, P]
    lib.mxfa_quantize_col32_row32.argtypes = [P, i64, i64, i32, P, i32, i32, P, P, P, P, P]
    lib.mxfa_quantize_e2m1.argtypes = [P, i64, i64, i32, P, P, P]
    lib.mxfa_quantize_e2m3.argtypes = [P, i64, i64, i32, P, P, P]
    lib.mxfa_e4m3_pack_patterns.argtypes = [ctypes.c_uint32, i64, i32, f32, P, P]
    lib.mxfa_padded_token_rows.argtypes = [P, i32]
    lib.mxfa_padded_token_rows.restype = i64
    lib.mxfa_fwd.argtypes = [ctypes.POINTER(_AttnArgs), P, P, P]
    lib.mxfa_fwd_p_scale.argtypes = [ctypes.POINTER(_AttnArgs), i32, P, P, P]
    lib.mxfa_fwd_mx_out.argtypes = [ctypes.POINTER(_AttnArgs), i32, P, P, P, P, P]
    lib.mxfa_bwd_workspace_size.argtypes = [ctypes.POINTER(_AttnArgs), i32]
    lib.mxfa_bwd_workspace_size.restype = ctypes.c_size_t
    lib.mxfa_bwd.argtypes = [ctypes.POINTER(_AttnArgs), _Mx, _Mx, P, P, P, i32, f32, P, ctypes.c_size_t, P, P, P, P]
    lib.mxfa_bwd_mx_out.argtypes = [ctypes.POINTER(_AttnArgs), _Mx, _Mx, P, P, P, i32, f32, P, ctypes.c_size_t, P, P, P,
                                    ctypes.POINTER(_GradMx), P]
    lib.mxfa_bwd_no_alloc.argtypes = [ctypes.POINTER(_AttnArgs), _Mx, _Mx, P, P, P, i32, f32, P, P, P, P]
    lib.mxfa_bwd_no_alloc_max_workspace.argtypes = []
    lib.mxfa_bwd_no_alloc_max_workspace.restype = ctypes.c_size_t
    lib.mxfa_rmsnorm_quantize.argtypes = [P, i64, i64, i32, P, f32, P, i32, i32, P, P, P, P]
    lib.mxfa_linear_quantize.argtypes = [_Mx, _Mx, i64, i32, i32, P, i32, i32, P, P, P, P]
    lib.mxfa_linear_bwd_data.argtypes = [_Mx, _Mx, i64, i32, i32, P, i32, i32, i32, P, P]
    lib.mxfa_linear_bwd_weight_workspace_size.argtypes = [i64, i32, i32, i32]
    lib.mxfa_linear_bwd_weight_workspace_size.restype = ctypes.c_size_t
    lib.mxfa_linear_bwd_weight.argtypes = [P, P, P, P, i64, i32, i32, P, i32, i32, P, ctypes.c_size_t, P, P]
    lib.mxfa_rmsnorm_bwd_workspace_size.argtypes = [i64, i32]
    lib.mxfa_rmsnorm_bwd_workspace_size.restype = ctypes.c_size_t
    lib.mxfa_rmsnorm_bwd.argtypes = [P, i64, i64, i32, P, f32, P, P, ctypes.c_size_t, P, P, P]
    lib.mxfa_status_string.argtypes = [i32]
    lib.mxfa_status_string.restype = ctypes.c_char_p
    lib.mxfa_last_error_message.argtypes = []
    lib.mxfa_last_error_message.restype = ctypes.c_char_p
    for n in ("mxfa_quantize", "mxfa_quantize_col32_row32", "mxfa_quantize_e2m1", "mxfa_quantize_e2m3", "mxfa_e4m3_pack_patterns", "mxfa_varlen_scale_scatter", "mxfa_fwd", "mxfa_fwd_p_scale", "mxfa_fwd_mx_out", "mxfa_bwd",
              "mxfa_bwd_mx_out", "mxfa_bwd_no_alloc", "mxfa_rmsnorm_quantize",
              "mxfa_linear_quantize", "mxfa_linear_bwd_data", "mxfa_linear_bwd_weight", "mxfa_rmsnorm_bwd"):
        getattr(lib, n).restype = i32
    _lib = lib
    return lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status, name):
    if status != 0:
        lib = _load()
        raise MxfaError(f"{name}: {lib.mxfa_status_string(status).decode()}: "
                        f"{lib.mxfa_last_error_message().decode()}")


# ------------------------------------------------------------------------------------------------
# The C ABI, one function per entry point
# ------------------------------------------------------------------------------------------------

def mxfa_status_string(status):
    return _load().mxfa_status_string(int(status)).decode()


def mxfa_last_error_message():
    return _load().mxfa_last_error_message().decode()


def mxfa_quantize(x, ld_x, T, C, cu_seqlens, nseq, max_seqlen, mode, data_out, scale_out, scale_t_out=None,
                  stream=None):
    _check(_load().mxfa_quantize(_ptr(x), ld_x, T, C, _ptr(cu_seqlens), nseq, max_seqlen, mode, _ptr(data_out),
                                 _ptr(scale_out), _ptr(scale_t_out), _stream(stream)), "mxfa_quantize")


def mxfa_quantize_col32_row32(x, ld_x, T, C, cu_seqlens, nseq, max_seqlen, data_col, scale_col, data_row, scale_row,
                              stream=None):
    _check(_load().mxfa_quantize_col32_row32(_ptr(x), ld_x, T, C, _ptr(cu_seqlens), nseq, max_seqlen, _ptr(data_col),
                                             _ptr(scale_col), _ptr(data_row), _ptr(scale_row), _stream(stream)),
           "mxfa_quantize_col32_row32")


def mxfa_e4m3_pack_patterns(first, n, variant, sc, out, stream=None):
    _check(_load().mxfa_e4m3_pack_patterns(first, n, variant, sc, _ptr(out), _stream(stream)), "mxfa_e4m3_pack_patterns")


def mxfa_quantize_e2m1(x, ld_x, T, C, data_out, scale_out, stream=None):
    _check(_load().mxfa_quantize_e2m1(_ptr(x), ld_x, T, C, _ptr(data_out), _ptr(scale_out), _stream(stream)),
           "mxfa_quantize_e2m1")


def mxfa_quantize_e2m3(x, ld_x, T, C, data_out, scale_out, stream=None):
    _check(_load().mxfa_quantize_e2m3(_ptr(x), ld_x, T, C, _ptr(data_out), _ptr(scale_out), _stream(stream)),
           "mxfa_quantize_e2m3")


def mxfa_varlen_scale_scatter(compact, cu_seqlens, nseq, max_seqlen, C, mode, padded_out, padded_rows, stream=None):
    _check(_load().mxfa_varlen_scale_scatter(_ptr(compact), _ptr(cu_seqlens), nseq, max_seqlen, C, mode,
                                             _ptr(padded_out), padded_rows, _stream(stream)),
           "mxfa_varlen_scale_scatter")


def mxfa_padded_token_rows(cu_seqlens_host):
    """cu_seqlens_host: a CPU int32 tensor or numpy array."""
    import numpy as np
    cu = np.ascontiguousarray(cu_seqlens_host.cpu().numpy() if hasattr(cu_seqlens_host, "cpu") else cu_seqlens_host,
                              dtype=np.int32)
    return int(_load().mxfa_padded_token_rows(cu.ctypes.data_as(ctypes.c_void_p), cu.size - 1))


class MxOperand:
    """Payload [T, C] uint8 tensor ([T, C/2] for E2M1) + scale uint8 tensor (layout per `mode`)."""

    def __init__(self, data, scale, mode, elem=E4M3):
        self.data, self.scale, self.mode, self.elem = data, scale, mode, elem

    def _c(self):
        return _Mx(_ptr(self.data), _ptr(self.scale), self.mode, self.elem)


class AttnArgs:
    """Python mirror of mxfa_attn_args."""

    def __init__(self, q, k, v, cu_seqlens_q, cu_seqlens_k, nseq, max_seqlen_q, max_seqlen_k, total_q, total_k,
                 num_heads, head_dim, softmax_scale, causal=False):
        self.q, self.k, self.v = q, k, v
        self.cu_seqlens_q, self.cu_seqlens_k = cu_seqlens_q, cu_seqlens_k
        self.nseq, self.max_seqlen_q, self.max_seqlen_k = nseq, max_seqlen_q, max_seqlen_k
        self.total_q, self.total_k = total_q, total_k
        self.num_heads, self.head_dim = num_heads, head_dim
        self.softmax_scale, self.causal = softmax_scale, causal

    def _c(self):
        return _AttnArgs(self.q._c(), self.k._c(), self.v._c(), _ptr(self.cu_seqlens_q), _ptr(self.cu_seqlens_k),
                         self.nseq, self.max_seqlen_q, self.max_seqlen_k, self.total_q, self.total_k,
                         self.num_heads, self.head_dim, self.softmax_scale, 1 if self.causal else 0)


def mxfa_fwd(args, o, lse, stream=None):
    a = args._c()
    _check(_load().mxfa_fwd(ctypes.byref(a), _ptr(o), _ptr(lse), _stream(stream)), "mxfa_fwd")


def mxfa_fwd_p_scale(args, p_scale, o, lse, stream=None):
    """p_scale: P_STATIC or P_BLOCK_DYNAMIC."""
    a = args._c()
    _check(_load().mxfa_fwd_p_scale(ctypes.byref(a), int(p_scale), _ptr(o), _ptr(lse), _stream(stream)),
           "mxfa_fwd_p_scale")


def mxfa_fwd_mx_out(args, p_scale, o, o_data, o_scale, lse, stream=None):
    """o (bf16) and o_data (E4M3, ROW32 codes in o_scale) may each be None, not both."""
    a = args._c()
    _check(_load().mxfa_fwd_mx_out(ctypes.byref(a), int(p_scale), _ptr(o), _ptr(o_data), _ptr(o_scale), _ptr(lse),
                                   _stream(stream)), "mxfa_fwd_mx_out")


def mxfa_bwd_workspace_size(args, dq_mode):
    """args: AttnArgs (or the ctypes struct)."""
    a = args._c() if hasattr(args, "_c") else args
    return int(_load().mxfa_bwd_workspace_size(ctypes.byref(a), dq_mode))


def mxfa_bwd(args, v_d, dout, o, dout_bf16, lse, dq_mode, dq_static_scale, workspace, workspace_bytes, dq, dk, dv,
             stream=None):
    a = args._c()
    _check(_load().mxfa_bwd(ctypes.byref(a), v_d._c(), dout._c(), _ptr(o), _ptr(dout_bf16), _ptr(lse), dq_mode,
                            dq_static_scale, _ptr(workspace), workspace_bytes, _ptr(dq), _ptr(dk), _ptr(dv),
                            _stream(stream)), "mxfa_bwd")


def mxfa_bwd_no_alloc(args, v_d, dout, o, dout_bf16, lse, dq_mode, dq_static_scale, dq, dk, dv, stream=None):
    """mxfa_bwd with the library's fixed per-GPU workspace array (no workspace argument)."""
    a = args._c()
    _check(_load().mxfa_bwd_no_alloc(ctypes.byref(a), v_d._c(), dout._c(), _ptr(o), _ptr(dout_bf16), _ptr(lse),
                                     dq_mode, dq_static_scale, _ptr(dq), _ptr(dk), _ptr(dv), _stream(stream)),
           "mxfa_bwd_no_alloc")


def mxfa_bwd_no_alloc_max_workspace():
    return int(_load().mxfa_bwd_no_alloc_max_workspace())


def mxfa_rmsnorm_quantize(x, ld_x, T, C, gamma, eps, cu_seqlens, nseq, max_seqlen, data_out, scale_out,
                          scale_t_out=None, stream=None):
    _check(_load().mxfa_rmsnorm_quantize(_ptr(x), ld_x, T, C, _ptr(gamma), eps, _ptr(cu_seqlens), nseq, max_seqlen,
                                         _ptr(data_out), _ptr(scale_out), _ptr(scale_t_out), _stream(stream)),
           "mxfa_rmsnorm_quantize")


# ------------------------------------------------------------------------------------------------
# Allocate-and-call helpers (outputs sized with torch on x's device)
# ------------------------------------------------------------------------------------------------

def _blockrows(lens):
    return int(sum((int(L) + 31) // 32 for L in lens))


def _lens(cu_host):
    cu = [int(v) for v in cu_host]
    return [cu[i + 1] - cu[i] for i in range(len(cu) - 1)]


def quantize(x_bf16, cu_host, cu_dev, mode, want_scale_t=False, stream=None):
    """x_bf16: torch.bfloat16 [T, C] on the GPU. Returns (data, scale, scale_t or None), compact layout."""
    T, C = x_bf16.shape
    lens = _lens(cu_host)
    dev = x_bf16.device
    data = torch.empty((T, C), dtype=torch.uint8, device=dev)
    nb = _blockrows(lens)
    shape = {ROW32: (T, C // 32), COL32: (nb, C), SQ32: (nb, C // 32)}[mode]
    scale = torch.empty(shape, dtype=torch.uint8, device=dev)
    scale_t = torch.empty((C // 32, nb), dtype=torch.uint8, device=dev) if (want_scale_t and mode == SQ32) else None
    mxfa_quantize(x_bf16, x_bf16.stride(0), T, C, cu_dev, len(lens), max(lens) if lens else 0, mode, data, scale,
                  scale_t, stream)
    return data, scale, scale_t


def quantize_e2m1(x_bf16, stream=None):
    """x_bf16: torch.bfloat16 [T, C] on the GPU. Returns (data [T, C/2], scale [T, C/32]): MXFP4 ROW32."""
    T, C = x_bf16.shape
    data = torch.empty((T, C // 2), dtype=torch.uint8, device=x_bf16.device)
    scale = torch.empty((T, C // 32), dtype=torch.uint8, device=x_bf16.device)
    mxfa_quantize_e2m1(x_bf16, x_bf16.stride(0), T, C, data, scale, stream)
    return data, scale


def quantize_e2m3(x_bf16, stream=None):
    """x_bf16: torch.bfloat16 [T, C] on the GPU. Returns (data [T, 3C/4], scale [T, C/32]): MXFP6 ROW32."""
    T, C = x_bf16.shape
    data = torch.empty((T, 3 * C // 4), dtype=torch.uint8, device=x_bf16.device)
    scale = torch.empty((T, C // 32), dtype=torch.uint8, device=x_bf16.device)
    mxfa_quantize_e2m3(x_bf16, x_bf16.stride(0), T, C, data, scale, stream)
    return data, scale


def scale_scatter(compact, cu_host, cu_dev, C, mode, stream=None):
    lens = _lens(cu_host)
    P = sum((L + 127) // 128 * 128 for L in lens)
    rows = P if mode == ROW32 else P // 32
    width = C if mode == COL32 else C // 32
    out = torch.empty((rows, width), dtype=torch.uint8, device=compact.device)
    mxfa_varlen_scale_scatter(compact, cu_dev, len(lens), max(lens) if lens else 0, C, mode, out, rows, stream)
    return out


def fwd_mx_out(args, stream=None, p_scale=P_STATIC, with_bf16=True):
    """Forward writing O as MXFP8 (ROW32 blocks along D). Returns (o bf16 or None, o_data u8 [T_q, H*D],
    o_scale u8 [T_q, H*D/32], lse fp32 [H, T_q])."""
    dev = args.q.data.device
    C = args.num_heads * args.head_dim
    o = torch.empty((args.total_q, C), dtype=torch.bfloat16, device=dev) if with_bf16 else None
    o_data = torch.empty((args.total_q, C), dtype=torch.uint8, device=dev)
    o_scale = torch.empty((args.total_q, C // 32), dtype=torch.uint8, device=dev)
    lse = torch.empty((args.num_heads, args.total_q), dtype=torch.float32, device=dev)
    mxfa_fwd_mx_out(args, p_scale, o, o_data, o_scale, lse, stream)
    return o, o_data, o_scale, lse


def fwd(args, stream=None, p_scale=P_STATIC):
    """Returns (o bf16 [T_q, H*D], lse fp32 [H, T_q])."""
    dev = args.q.data.device
    o = torch.empty((args.total_q, args.num_heads * args.head_dim), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((args.num_heads, args.total_q), dtype=torch.float32, device=dev)
    if p_scale == P_STATIC:
        mxfa_fwd(args, o, lse, stream)
    else:
        mxfa_fwd_p_scale(args, p_scale, o, lse, stream)
    return o, lse


def bwd(args, v_d, dout, o, dout_bf16, lse, dq_mode=DQ_FP32, dq_static_scale=1.0, workspace=None, stream=None):
    """Returns (dq, dk, dv) bf16."""
    dev = args.q.data.device
    C = args.num_heads * args.head_dim
    need = mxfa_bwd_workspace_size(args, dq_mode)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    dq = torch.empty((args.total_q, C), dtype=torch.bfloat16, device=dev)
    dk = torch.empty((args.total_k, C), dtype=torch.bfloat16, device=dev)
    dv = torch.empty((args.total_k, C), dtype=torch.bfloat16, device=dev)
    mxfa_bwd(args, v_d, dout, o, dout_bf16, lse, dq_mode, dq_static_scale, workspace, workspace.numel(), dq, dk, dv,
             stream)
    return dq, dk, dv


def mxfa_bwd_mx_out(args, v_d, dout, o, dout_bf16, lse, dq_mode, dq_static_scale, workspace, workspace_bytes, dq, dk,
                    dv, mx_out, stream=None):
    """dq, dk, dv: bf16 tensors or None (all or none); mx_out: sequence of the six tensors
    (dq, dq_scale, dk, dk_scale, dv, dv_scale), optionally followed by the three transposed code grids
    (dq_scale_t, dk_scale_t, dv_scale_t; each may be None), or None."""
    a = args._c()
    g = ctypes.byref(_GradMx(*[_ptr(t) for t in mx_out])) if mx_out is not None else None
    _check(_load().mxfa_bwd_mx_out(ctypes.byref(a), v_d._c(), dout._c(), _ptr(o), _ptr(dout_bf16), _ptr(lse), dq_mode,
                                   dq_static_scale, _ptr(workspace), workspace_bytes, _ptr(dq), _ptr(dk), _ptr(dv), g,
                                   _stream(stream)), "mxfa_bwd_mx_out")


def bwd_mx_out(args, v_d, dout, o, dout_bf16, lse, cu_q_host, cu_k_host, dq_mode=DQ_FP32, dq_static_scale=1.0,
               with_bf16=True, stream=None):
    """Backward with MXFP8 gradients (SQ32, compact codes). Returns ((dq, dk, dv) bf16 or None,
    (dq, dq_scale, dk, dk_scale, dv, dv_scale))."""
    dev = args.q.data.device
    C = args.num_heads * args.head_dim
    workspace = torch.empty(mxfa_bwd_workspace_size(args, dq_mode), dtype=torch.uint8, device=dev)
    nbq, nbk = _blockrows(_lens(cu_q_host)), _blockrows(_lens(cu_k_host))
    u8 = lambda *shape: torch.empty(shape, dtype=torch.uint8, device=dev)
    mx_out = (u8(args.total_q, C), u8(nbq, C // 32), u8(args.total_k, C), u8(nbk, C // 32), u8(args.total_k, C),
              u8(nbk, C // 32))
    bf = None
    if with_bf16:
        bf = (torch.empty((args.total_q, C), dtype=torch.bfloat16, device=dev),
              torch.empty((args.total_k, C), dtype=torch.bfloat16, device=dev),
              torch.empty((args.total_k, C), dtype=torch.bfloat16, device=dev))
    mxfa_bwd_mx_out(args, v_d, dout, o, dout_bf16, lse, dq_mode, dq_static_scale, workspace, workspace.numel(),
                    *(bf if bf else (None, None, None)), mx_out, stream)
    return bf, mx_out


def rmsnorm_quantize(x_bf16, gamma, eps, cu_host, cu_dev, want_scale_t=True, stream=None):
    T, C = x_bf16.shape
    lens = _lens(cu_host)
    dev = x_bf16.device
    nb = _blockrows(lens)
    data = torch.empty((T, C), dtype=torch.uint8, device=dev)
    scale = torch.empty((nb, C // 32), dtype=torch.uint8, device=dev)
    scale_t = torch.empty((C // 32, nb), dtype=torch.uint8, device=dev) if want_scale_t else None
    mxfa_rmsnorm_quantize(x_bf16, x_bf16.stride(0), T, C, gamma, eps, cu_dev, len(lens), max(lens) if lens else 0,
                          data, scale, scale_t, stream)
    return data, scale, scale_t


def mxfa_linear_quantize(x, w, T, C_in, C_out, cu_seqlens, nseq, max_seqlen, data_out, scale_out, scale_t_out=None,
                         stream=None):
    """x, w: MxOperand (x SQ32 or ROW32 compact scales, w ROW32)."""
    _check(_load().mxfa_linear_quantize(x._c(), w._c(), T, C_in, C_out, _ptr(cu_seqlens), nseq, max_seqlen,
                                        _ptr(data_out), _ptr(scale_out), _ptr(scale_t_out), _stream(stream)),
           "mxfa_linear_quantize")


def linear_quantize(x, w, cu_host, cu_dev, want_scale_t=True, stream=None):
    """Projection + SQ32 quantize: returns (data [T, C_out], scale [NB, C_out/32], scale_t or None)."""
    T, C_in = x.data.shape
    C_out = w.data.shape[0]
    lens = _lens(cu_host)
    dev = x.data.device
    nb = _blockrows(lens)
    data = torch.empty((T, C_out), dtype=torch.uint8, device=dev)
    scale = torch.empty((nb, C_out // 32), dtype=torch.uint8, device=dev)
    scale_t = torch.empty((C_out // 32, nb), dtype=torch.uint8, device=dev) if want_scale_t else None
    mxfa_linear_quantize(x, w, T, C_in, C_out, cu_dev, len(lens), max(lens) if lens else 0, data, scale, scale_t,
                         stream)
    return data, scale, scale_t


def mxfa_linear_bwd_data(dy, wt, T, C_out, C_in, cu_seqlens, nseq, max_seqlen, accumulate, dx, stream=None):
    """dy: MxOperand [T, C_out] (SQ32 or ROW32 compact scales); wt: MxOperand W^T [C_in, C_out] ROW32;
    accumulate 1 adds to dx."""
    _check(_load().mxfa_linear_bwd_data(dy._c(), wt._c(), T, C_out, C_in, _ptr(cu_seqlens), nseq, max_seqlen,
                                        int(accumulate), _ptr(dx), _stream(stream)), "mxfa_linear_bwd_data")


def mxfa_linear_bwd_weight_workspace_size(T, nseq, C_out, C_in):
    return int(_load().mxfa_linear_bwd_weight_workspace_size(T, nseq, C_out, C_in))


def mxfa_linear_bwd_weight(dy, dy_scale_t, x, x_scale_t, T, C_out, C_in, cu_seqlens, nseq, max_seqlen, workspace,
                           workspace_bytes, dw, stream=None):
    _check(_load().mxfa_linear_bwd_weight(_ptr(dy), _ptr(dy_scale_t), _ptr(x), _ptr(x_scale_t), T, C_out, C_in,
                                          _ptr(cu_seqlens), nseq, max_seqlen, _ptr(workspace), workspace_bytes,
                                          _ptr(dw), _stream(stream)), "mxfa_linear_bwd_weight")


def mxfa_rmsnorm_bwd_workspace_size(T, C):
    return int(_load().mxfa_rmsnorm_bwd_workspace_size(T, C))


def mxfa_rmsnorm_bwd(x, ld_x, T, C, gamma, eps, dy, workspace, workspace_bytes, dx, dgamma, stream=None):
    _check(_load().mxfa_rmsnorm_bwd(_ptr(x), ld_x, T, C, _ptr(gamma), eps, _ptr(dy), _ptr(workspace), workspace_bytes,
                                    _ptr(dx), _ptr(dgamma), _stream(stream)), "mxfa_rmsnorm_bwd")


def linear_bwd_data(dy, wt, cu_host, cu_dev, dx=None, stream=None):
    """dX = dY W as bf16 [T, C_in] (dy: MxOperand [T, C_out]; wt: MxOperand W^T [C_in, C_out] ROW32); with
    dx given, the product is added to it."""
    T, C_out = dy.data.shape
    C_in = wt.data.shape[0]
    lens = _lens(cu_host)
    acc = dx is not None
    if dx is None:
        dx = torch.empty((T, C_in), dtype=torch.bfloat16, device=dy.data.device)
    mxfa_linear_bwd_data(dy, wt, T, C_out, C_in, cu_dev, len(lens), max(lens) if lens else 0, acc, dx, stream)
    return dx


def linear_bwd_weight(dy, dy_scale_t, x, x_scale_t, cu_host, cu_dev, workspace=None, stream=None):
    """dW = dY^T X as FP32 [C_out, C_in] from SQ32 payloads and their transposed scale grids."""
    T, C_out = dy.shape
    C_in = x.shape[1]
    lens = _lens(cu_host)
    need = mxfa_linear_bwd_weight_workspace_size(T, len(lens), C_out, C_in)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dy.device)
    dw = torch.empty((C_out, C_in), dtype=torch.float32, device=dy.device)
    mxfa_linear_bwd_weight(dy, dy_scale_t, x, x_scale_t, T, C_out, C_in, cu_dev, len(lens), max(lens) if lens else 0,
                           workspace, workspace.numel(), dw, stream)
    return dw


def rmsnorm_bwd(x_bf16, gamma, eps, dy_bf16, workspace=None, stream=None):
    """RMSNorm backward: returns (dx bf16 [T, C], dgamma FP32 [C])."""
    T, C = x_bf16.shape
    need = mxfa_rmsnorm_bwd_workspace_size(T, C)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x_bf16.device)
    dx = torch.empty((T, C), dtype=torch.bfloat16, device=x_bf16.device)
    dg = torch.empty(C, dtype=torch.float32, device=x_bf16.device)
    mxfa_rmsnorm_bwd(x_bf16, x_bf16.stride(0), T, C, gamma, eps, dy_bf16, workspace, workspace.numel(), dx, dg, stream)
    return dx, dg
