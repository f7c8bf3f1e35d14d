"""Python binding of the CPU oracle (liboracle: oracle/mx_oracle.cpp).

TEST INFRASTRUCTURE ONLY: imported by the test suite, by the smoke check and by the
benchmark's CPU-baseline leg. The product path never imports this package.

All arrays are numpy, host memory. Layouts follow the compact layouts of the C source:
payload [T, C] uint8; ROW32 scales [T, C/32]; COL32 scales [NB, C]; SQ32 scales [NB, C/32]
(+ transposed [C/32, NB]); NB = sum over sequences of ceil(L/32).
"""
import ctypes
import os
import subprocess

import numpy as np

ROW32, COL32, SQ32 = 0, 1, 2
_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mx_oracle.cpp")
_LIB_PATH = os.path.join(_HERE, "libmxoracle.so")
_lib = None


def build():
    """Compile the oracle with g++ (no HIP headers, no GPU code)."""
    cmd = ["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fPIC", "-shared", "-pthread",
           _SRC, "-o", _LIB_PATH]
    subprocess.run(cmd, check=True)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i64, i32, f32, f64 = ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_double
    lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_decode.restype = f64
    lib.orc_e4m3_encode.argtypes = [f64]
    lib.orc_e4m3_encode.restype = ctypes.c_uint8
    lib.orc_e8m0_code.argtypes = [f64]
    lib.orc_e8m0_code.restype = i32
    lib.orc_e8m0_value.argtypes = [i32]
    lib.orc_e8m0_value.restype = f64
    lib.orc_fp16_round.argtypes = [f64]
    lib.orc_fp16_round.restype = f64
    lib.orc_f32_to_bf16.argtypes = [f32]
    lib.orc_f32_to_bf16.restype = ctypes.c_uint16
    lib.orc_e4m3_encode_array.argtypes = [P, i64, P]
    lib.orc_e4m3_encode_array.restype = None
    lib.orc_num_blockrows.argtypes = [P, i32]
    lib.orc_num_blockrows.restype = i64
    lib.orc_padded_rows.argtypes = [P, i32]
    lib.orc_padded_rows.restype = i64
    lib.orc_quantize_bf16.argtypes = [P, i64, i64, i32, P, i32, i32, P, P, P]
    lib.orc_quantize_f32.argtypes = [P, i64, i32, P, i32, i32, P, P, P]
    lib.orc_dequantize.argtypes = [P, P, i64, i32, P, i32, i32, P]
    lib.orc_scale_scatter.argtypes = [P, P, i32, i32, i32, P, i64]
    lib.orc_attn_fwd_f64.argtypes = [P, P, P, P, P, i32, i32, i32, f32, i32, i32, i32, P, P, P, i32]
    lib.orc_attn_fwd_mx.argtypes = [P, P, i32, P, P, i32, P, P, i32, P, P, i32, i32, i32, f32, i32, i32, P, P, P, i32]
    lib.orc_attn_bwd_f64.argtypes = [P, P, P, P, P, P, P, P, P, i32, i32, i32, f32, i32, i32, i32, f32,
                                     P, P, P, P, P, P, P, i32]
    lib.orc_attn_bwd_mx.argtypes = [P, P, P, P, P, P, i32, P, P, P, P, P, P, P, i32, i32, i32, f32, i32, i32, f32,
                                    P, P, P, P, P, P, P, i32]
    lib.orc_rmsnorm_quantize.argtypes = [P, i64, i64, i32, P, f32, P, i32, P, P, P, P]
    lib.orc_linear_quantize.argtypes = [P, P, i32, P, P, i64, i32, i32, P, i32, P, P, P, P, i32]
    lib.orc_linear_bwd_data.argtypes = [P, P, P, P, i64, i32, i32, P, i32, P, P, P, i32]
    lib.orc_linear_bwd_weight.argtypes = [P, P, P, P, i64, i32, i32, P, i32, P, i32]
    lib.orc_rmsnorm_bwd.argtypes = [P, i64, i64, i32, P, f32, P, P, P, P]
    for name in ["orc_quantize_bf16", "orc_quantize_f32", "orc_dequantize", "orc_scale_scatter",
                 "orc_attn_fwd_f64", "orc_attn_fwd_mx", "orc_attn_bwd_f64", "orc_attn_bwd_mx",
                 "orc_rmsnorm_quantize", "orc_linear_quantize"]:
        getattr(lib, name).restype = i32
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"oracle {name}: invalid arguments")


def default_threads():
    """At most 16 threads: the CPU share of one GPU on the machines this runs on, whatever the core
    count the OS reports."""
    return max(1, min(os.cpu_count() or 1, 16))


# ---- scalars ------------------------------------------------------------------------------

def e4m3_decode(code):
    return _load().orc_e4m3_decode(int(code))


def e4m3_encode(v):
    return int(_load().orc_e4m3_encode(float(v)))


def e4m3_encode_array(x):
    x = _c(x, np.float32).ravel()
    out = np.empty(x.size, np.uint8)
    _load().orc_e4m3_encode_array(_p(x), x.size, _p(out))
    return out


def e8m0_code(amax):
    return int(_load().orc_e8m0_code(float(amax)))


def e8m0_value(code):
    return _load().orc_e8m0_value(int(code))


def fp16_round(v):
    return _load().orc_fp16_round(float(v))


def f32_to_bf16(f):
    return int(_load().orc_f32_to_bf16(float(f)))


# ---- layouts ------------------------------------------------------------------------------

def num_blockrows(cu):
    cu = _c(cu, np.int32)
    return int(_load().orc_num_blockrows(_p(cu), cu.size - 1))


def padded_rows(cu):
    cu = _c(cu, np.int32)
    return int(_load().orc_padded_rows(_p(cu), cu.size - 1))


def scale_shape(mode, T, C, cu):
    nb = num_blockrows(cu)
    return {ROW32: (T, C // 32), COL32: (nb, C), SQ32: (nb, C // 32)}[mode]


# ---- quantize / dequantize / scatter -------------------------------------------------------

def quantize(x, cu, mode):
    """x: [T, C] as uint16 (bf16 bits) or float32. Returns (data, scale, scale_t or None)."""
    lib = _load()
    cu = _c(cu, np.int32)
    T, C = x.shape
    data = np.empty((T, C), np.uint8)
    scale = np.empty(scale_shape(mode, T, C, cu), np.uint8)
    scale_t = np.empty((C // 32, num_blockrows(cu)), np.uint8) if mode == SQ32 else None
    if x.dtype == np.uint16:
        xs = _c(x, np.uint16)
        rc = lib.orc_quantize_bf16(_p(xs), C, T, C, _p(cu), cu.size - 1, mode, _p(data), _p(scale), _p(scale_t))
    else:
        xs = _c(x, np.float32)
        rc = lib.orc_quantize_f32(_p(xs), T, C, _p(cu), cu.size - 1, mode, _p(data), _p(scale), _p(scale_t))
    _check(rc, "quantize")
    return data, scale, scale_t


def dequantize(data, scale, cu, mode):
    lib = _load()
    cu = _c(cu, np.int32)
    data = _c(data, np.uint8)
    scale = _c(scale, np.uint8)
    T, C = data.shape
    out = np.empty((T, C), np.float64)
    _check(lib.orc_dequantize(_p(data), _p(scale), T, C, _p(cu), cu.size - 1, mode, _p(out)), "dequantize")
    return out


def scale_scatter(compact, cu, C, mode):
    lib = _load()
    cu = _c(cu, np.int32)
    compact = _c(compact, np.uint8)
    P = padded_rows(cu)
    rows = P if mode == ROW32 else P // 32
    width = C if mode == COL32 else C // 32
    out = np.empty((rows, width), np.uint8)
    _check(lib.orc_scale_scatter(_p(compact), _p(cu), cu.size - 1, C, mode, _p(out), rows), "scale_scatter")
    return out


# ---- attention -----------------------------------------------------------------------------

P_NONE, P_STATIC, P_DYNAMIC = 0, 1, 2  # P quantization modes of the forward

def attn_fwd_f64(q, k, v, cu_q, cu_k, H, D, softmax_scale, causal=False, quant_p=True, kv_tile=128, nthreads=None):
    """q, k, v: float64 [T, H*D]. Returns (o_bf16 uint16 [Tq, H*D], o_f32 [Tq, H*D], lse [H, Tq]).
    quant_p: P_NONE / False (no P quantization), P_STATIC / True (scale 2^-8 on every block) or
    P_DYNAMIC (each 32-key block scaled by the MX rule on its largest P)."""
    lib = _load()
    cu_q, cu_k = _c(cu_q, np.int32), _c(cu_k, np.int32)
    q, k, v = _c(q, np.float64), _c(k, np.float64), _c(v, np.float64)
    Tq = q.shape[0]
    o16 = np.empty((Tq, H * D), np.uint16)
    o32 = np.empty((Tq, H * D), np.float32)
    lse = np.empty((H, Tq), np.float32)
    rc = lib.orc_attn_fwd_f64(_p(q), _p(k), _p(v), _p(cu_q), _p(cu_k), cu_q.size - 1, H, D, softmax_scale,
                              int(causal), int(quant_p), kv_tile, _p(o16), _p(o32), _p(lse),
                              nthreads or default_threads())
    _check(rc, "attn_fwd_f64")
    return o16, o32, lse


def attn_fwd_mx(q, q_scale, q_mode, k, k_scale, k_mode, v, v_scale, v_mode, cu_q, cu_k, H, D, softmax_scale,
                causal=False, p_scale=1, nthreads=None):
    """MX inputs in compact layouts. Returns (o_bf16 [Tq, H*D] uint16, o_f32, lse [H, Tq]).
    p_scale: P_STATIC (1) or P_DYNAMIC (2), as for attn_fwd_f64."""
    lib = _load()
    cu_q, cu_k = _c(cu_q, np.int32), _c(cu_k, np.int32)
    arrs = [_c(a, np.uint8) for a in (q, q_scale, k, k_scale, v, v_scale)]
    Tq = arrs[0].shape[0]
    o16 = np.empty((Tq, H * D), np.uint16)
    o32 = np.empty((Tq, H * D), np.float32)
    lse = np.empty((H, Tq), np.float32)
    rc = lib.orc_attn_fwd_mx(_p(arrs[0]), _p(arrs[1]), q_mode, _p(arrs[2]), _p(arrs[3]), k_mode, _p(arrs[4]),
                             _p(arrs[5]), v_mode, _p(cu_q), _p(cu_k), cu_q.size - 1, H, D, softmax_scale,
                             int(causal), int(p_scale), _p(o16), _p(o32), _p(lse), nthreads or default_threads())
    _check(rc, "attn_fwd_mx")
    return o16, o32, lse


def attn_bwd_f64(q, k, v, dO_mm, o_delta, do_delta, lse, cu_q, cu_k, H, D, softmax_scale, causal=False,
                 quant=True, dq_mode=0, dq_sigma=1.0, nthreads=None):
    """Double inputs [T, H*D]; lse [H, Tq] fp32. Returns dict of float32 dq, dk, dv (+ bf16 and overflow)."""
    lib = _load()
    cu_q, cu_k = _c(cu_q, np.int32), _c(cu_k, np.int32)
    q, k, v, dO_mm, o_delta, do_delta = (_c(a, np.float64) for a in (q, k, v, dO_mm, o_delta, do_delta))
    lse = _c(lse, np.float32)
    Tq, Tk = q.shape[0], k.shape[0]
    out = {n: np.empty(s, t) for n, s, t in [
        ("dq", (Tq, H * D), np.uint16), ("dk", (Tk, H * D), np.uint16), ("dv", (Tk, H * D), np.uint16),
        ("dq_f", (Tq, H * D), np.float32), ("dk_f", (Tk, H * D), np.float32), ("dv_f", (Tk, H * D), np.float32)]}
    ovf = ctypes.c_int(0)
    rc = lib.orc_attn_bwd_f64(_p(q), _p(k), _p(v), _p(dO_mm), _p(o_delta), _p(do_delta), _p(lse), _p(cu_q),
                              _p(cu_k), cu_q.size - 1, H, D, softmax_scale, int(causal), int(quant), dq_mode,
                              dq_sigma, _p(out["dq"]), _p(out["dk"]), _p(out["dv"]), _p(out["dq_f"]),
                              _p(out["dk_f"]), _p(out["dv_f"]), ctypes.addressof(ovf), nthreads or default_threads())
    _check(rc, "attn_bwd_f64")
    out["overflow"] = ovf.value
    return out


def attn_bwd_mx(q, q_scale, k, k_scale, v, v_scale, v_mode, dO, dO_scale, o_bf16, do_bf16, lse, cu_q, cu_k, H, D,
                softmax_scale, causal=False, dq_mode=0, dq_sigma=1.0, nthreads=None):
    lib = _load()
    cu_q, cu_k = _c(cu_q, np.int32), _c(cu_k, np.int32)
    u8 = [_c(a, np.uint8) for a in (q, q_scale, k, k_scale, v, v_scale, dO, dO_scale)]
    o_bf16, do_bf16 = _c(o_bf16, np.uint16), _c(do_bf16, np.uint16)
    lse = _c(lse, np.float32)
    Tq, Tk = u8[0].shape[0], u8[2].shape[0]
    out = {n: np.empty(s, t) for n, s, t in [
        ("dq", (Tq, H * D), np.uint16), ("dk", (Tk, H * D), np.uint16), ("dv", (Tk, H * D), np.uint16),
        ("dq_f", (Tq, H * D), np.float32), ("dk_f", (Tk, H * D), np.float32), ("dv_f", (Tk, H * D), np.float32)]}
    ovf = ctypes.c_int(0)
    rc = lib.orc_attn_bwd_mx(_p(u8[0]), _p(u8[1]), _p(u8[2]), _p(u8[3]), _p(u8[4]), _p(u8[5]), v_mode, _p(u8[6]),
                             _p(u8[7]), _p(o_bf16), _p(do_bf16), _p(lse), _p(cu_q), _p(cu_k), cu_q.size - 1, H, D,
                             softmax_scale, int(causal), dq_mode, dq_sigma, _p(out["dq"]), _p(out["dk"]),
                             _p(out["dv"]), _p(out["dq_f"]), _p(out["dk_f"]), _p(out["dv_f"]), ctypes.addressof(ovf),
                             nthreads or default_threads())
    _check(rc, "attn_bwd_mx")
    out["overflow"] = ovf.value
    return out


def rmsnorm_quantize(x_bf16, gamma, eps, cu):
    """x_bf16: uint16 [T, C]. Returns (data, scale [NB, C/32], scale_t [C/32, NB], y float32 [T, C])."""
    lib = _load()
    cu = _c(cu, np.int32)
    x = _c(x_bf16, np.uint16)
    gamma = _c(gamma, np.float32)
    T, C = x.shape
    nb = num_blockrows(cu)
    data = np.empty((T, C), np.uint8)
    scale = np.empty((nb, C // 32), np.uint8)
    scale_t = np.empty((C // 32, nb), np.uint8)
    y = np.empty((T, C), np.float32)
    rc = lib.orc_rmsnorm_quantize(_p(x), C, T, C, _p(gamma), eps, _p(cu), cu.size - 1, _p(data), _p(scale),
                                  _p(scale_t), _p(y))
    _check(rc, "rmsnorm_quantize")
    return data, scale, scale_t, y


def linear_quantize(x, x_scale, w, w_scale, cu, x_mode=SQ32, nthreads=None):
    """x [T, C_in] payload with SQ32 compact (or ROW32) scales; w [C_out, C_in] payload with ROW32 scales.
    Returns (data [T, C_out], scale [NB, C_out/32], scale_t [C_out/32, NB], y float32 [T, C_out])."""
    lib = _load()
    cu = _c(cu, np.int32)
    x, xs, w, ws = (_c(a, np.uint8) for a in (x, x_scale, w, w_scale))
    T, C_in = x.shape
    C_out = w.shape[0]
    nb = num_blockrows(cu)
    data = np.empty((T, C_out), np.uint8)
    scale = np.empty((nb, C_out // 32), np.uint8)
    scale_t = np.empty((C_out // 32, nb), np.uint8)
    y = np.empty((T, C_out), np.float32)
    rc = lib.orc_linear_quantize(_p(x), _p(xs), int(x_mode), _p(w), _p(ws), T, C_in, C_out, _p(cu), cu.size - 1, _p(data),
                                 _p(scale), _p(scale_t), _p(y), nthreads or default_threads())
    _check(rc, "linear_quantize")
    return data, scale, scale_t, y


def linear_bwd_data(dy, dy_scale, wt, wt_scale, cu, dx_in=None, nthreads=None):
    """dX = dY W (+ dx_in): dy [T, C_out] SQ32 payload with compact scales [NB, C_out/32]; wt = W^T
    [C_in, C_out] payload with ROW32 scales [C_in, C_out/32]; dx_in optional bf16 bits [T, C_in] the
    product is added to. Returns (dx bf16 bits uint16 [T, C_in], dx float32)."""
    lib = _load()
    cu = _c(cu, np.int32)
    dy, dys, wt, wts = (_c(a, np.uint8) for a in (dy, dy_scale, wt, wt_scale))
    T, C_out = dy.shape
    C_in = wt.shape[0]
    dxi = None if dx_in is None else _c(dx_in, np.uint16)
    dx = np.empty((T, C_in), np.uint16)
    dxf = np.empty((T, C_in), np.float32)
    rc = lib.orc_linear_bwd_data(_p(dy), _p(dys), _p(wt), _p(wts), T, C_out, C_in, _p(cu), cu.size - 1, _p(dxi),
                                 _p(dx), _p(dxf), nthreads or default_threads())
    _check(rc, "linear_bwd_data")
    return dx, dxf


def linear_bwd_weight(dy, dy_scale_t, x, x_scale_t, cu, nthreads=None):
    """dW = dY^T X over all tokens: dy [T, C_out] and x [T, C_in] SQ32 payloads with their transposed scale
    grids [C_out/32, NB] and [C_in/32, NB]. Returns dw float32 [C_out, C_in]."""
    lib = _load()
    cu = _c(cu, np.int32)
    dy, dyst, x, xst = (_c(a, np.uint8) for a in (dy, dy_scale_t, x, x_scale_t))
    T, C_out = dy.shape
    C_in = x.shape[1]
    dw = np.empty((C_out, C_in), np.float32)
    rc = lib.orc_linear_bwd_weight(_p(dy), _p(dyst), _p(x), _p(xst), T, C_out, C_in, _p(cu), cu.size - 1, _p(dw),
                                   nthreads or default_threads())
    _check(rc, "linear_bwd_weight")
    return dw


def rmsnorm_bwd(x_bf16, gamma, eps, dy_bf16):
    """x_bf16, dy_bf16: uint16 [T, C]. Returns (dx bf16 bits uint16 [T, C], dx float32, dgamma float32 [C])."""
    lib = _load()
    x = _c(x_bf16, np.uint16)
    dy = _c(dy_bf16, np.uint16)
    gamma = _c(gamma, np.float32)
    T, C = x.shape
    dx = np.empty((T, C), np.uint16)
    dxf = np.empty((T, C), np.float32)
    dg = np.empty(C, np.float32)
    rc = lib.orc_rmsnorm_bwd(_p(x), C, T, C, _p(gamma), eps, _p(dy), _p(dx), _p(dxf), _p(dg))
    _check(rc, "rmsnorm_bwd")
    return dx, dxf, dg
