"""CPU oracle for the decode-time ternary MoE FFN -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import this package.
The product library (``ternary_weight_moe_amd``) never imports it and shares no code with it.

The arithmetic lives in ``tw_oracle.c`` (plain C, doubles for the truth mode, a fixed fp32
operation sequence for the int8 spec mode); this module only marshals numpy arrays into it.
Inputs are taken as numpy arrays or CPU torch tensors; bf16/fp32 values are widened to float64
exactly before the call.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tw_oracle.c")
# TW_ORACLE_LIB: another build of the same source (for instance one with sanitizers)
_LIB = os.environ.get("TW_ORACLE_LIB") or os.path.join(_HERE, "libtw_oracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2 -ffp-contract=off -fopenmp)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-std=c11",
               "-Wall", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _P(t):
    return C.POINTER(t)


class _Layer(C.Structure):
    _fields_ = [("d_model", C.c_int32), ("d_ff", C.c_int32), ("n_experts", C.c_int32),
                ("top_k", C.c_int32), ("pre_rmsnorm", C.c_int32),
                ("w_router", _P(C.c_double)), ("t_gate", _P(C.c_uint8)), ("t_up", _P(C.c_uint8)),
                ("t_down", _P(C.c_uint8)), ("s_gate", _P(C.c_double)), ("s_up", _P(C.c_double)),
                ("s_down", _P(C.c_double))]


class _LayerI8(C.Structure):
    _fields_ = [("d_model", C.c_int32), ("d_ff", C.c_int32), ("n_experts", C.c_int32),
                ("top_k", C.c_int32), ("t_gate", _P(C.c_uint8)), ("t_up", _P(C.c_uint8)),
                ("t_down", _P(C.c_uint8)), ("s_gate", _P(C.c_float)), ("s_up", _P(C.c_float)),
                ("s_down", _P(C.c_float))]


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build(force=False)
            L = C.CDLL(_LIB)
            i64, i32, u8p, i8p = C.c_int64, C.c_int32, _P(C.c_uint8), _P(C.c_int8)
            dp, fp, ip = _P(C.c_double), _P(C.c_float), _P(C.c_int32)
            sig = {
                "or_bad_codes": (i64, []),
                "or_reset_bad_codes": (None, []),
                "or_pack": (i64, [i8p, i64, i64, u8p]),
                "or_unpack": (i64, [u8p, i64, i64, i8p]),
                "or_ternary_gemv": (None, [u8p, i64, i64, dp, dp, dp]),
                "or_f64_to_bf16": (C.c_uint16, [C.c_double]),
                "or_round_bf16_array": (None, [dp, i64, _P(C.c_uint16)]),
                "or_round_f32_array": (None, [dp, i64, fp]),
                "or_route": (None, [_P(_Layer), dp, i64, ip, dp, dp, i32]),
                "or_ffn_token": (None, [_P(_Layer), dp, ip, dp, dp]),
                "or_moe_layer": (None, [_P(_Layer), dp, i64, dp, ip, dp, dp, i32]),
                "or_decode_stack": (None, [_P(_Layer), i32, dp, i32, dp, dp, ip, dp, dp]),
                "or_dense_ffn_token": (None, [_P(_Layer), dp, ip, dp, dp]),
                "or_spec_expf": (C.c_float, [C.c_float]),
                "or_quant_absmax": (None, [fp, i64, i8p, fp]),
                "or_ffn_token_i8": (None, [_P(_LayerI8), fp, ip, fp, fp, i8p, fp, ip, ip, i8p, fp,
                                           ip, fp]),
                "or_ffn_batch_i8": (None, [_P(_LayerI8), fp, i64, ip, fp, fp, i32]),
                "or_quantize_absmean": (C.c_int, [fp, i64, i64, i8p, fp]),
                "or_pack3": (i64, [i8p, i64, i64, i64, u8p]),
                "or_unpack3": (i64, [u8p, i64, i64, i64, i8p]),
                "or_gemv_i8": (None, [i8p, fp, i64, i64, i8p, C.c_float, fp]),
                "or_attention_decode": (None, [dp, dp, dp, i64, i32, i32, i32, dp]),
                "or_flash_head": (None, [fp, i32, u8p, fp, i32, dp, ip, i32, i32, ip, ip, dp, fp]),
            }
            for name, (res, args) in sig.items():
                f = getattr(L, name)
                f.restype = res
                f.argtypes = args
            _lib = L
        return _lib


# ---- marshalling helpers -------------------------------------------------------------------

def _np(a, dtype):
    """numpy copy/view of a numpy array or CPU torch tensor, widened exactly to ``dtype``."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu()
            if a.dtype == torch.bfloat16:
                a = a.float()
            a = a.numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(a), dtype=dtype)


def _ptr(a, ctype):
    return a.ctypes.data_as(_P(ctype)) if a is not None else None


def _check_codes():
    n = lib().or_bad_codes()
    if n:
        lib().or_reset_bad_codes()
        raise ValueError("oracle met %d invalid 2-bit codes (11)" % n)


# ---- packing / rounding ------------------------------------------------------------------------

def pack(w) -> tuple[np.ndarray, int]:
    """int8 [..., cols] -> packed uint8 [..., ceil(cols/4)], number of values outside {-1,0,1}."""
    w = _np(w, np.int8)
    cols = w.shape[-1]
    rows = int(np.prod(w.shape[:-1])) if w.ndim > 1 else 1
    out = np.empty(w.shape[:-1] + ((cols + 3) // 4,), dtype=np.uint8)
    bad = lib().or_pack(_ptr(w, C.c_int8), rows, cols, _ptr(out, C.c_uint8))
    return out, int(bad)


def quantize_absmean(w) -> tuple[np.ndarray, np.ndarray]:
    """float [..., cols] (fp32 or bf16 values) -> (int8 codes in {-1,0,1} [..., cols], fp32 scales
    [...]): per-row absmean quantisation, tw_oracle.c."""
    w = _np(w, np.float32)
    cols = w.shape[-1]
    rows = int(np.prod(w.shape[:-1])) if w.ndim > 1 else 1
    t = np.empty(w.shape, dtype=np.int8)
    s = np.empty(w.shape[:-1] if w.ndim > 1 else (1,), dtype=np.float32)
    if lib().or_quantize_absmean(_ptr(w, C.c_float), rows, cols, _ptr(t, C.c_int8),
                                 _ptr(s, C.c_float)) != 0:
        raise ValueError("cols must be >= 0")
    return t, s


def unpack(packed, cols: int) -> tuple[np.ndarray, int]:
    p = _np(packed, np.uint8)
    rows = int(np.prod(p.shape[:-1])) if p.ndim > 1 else 1
    out = np.empty(p.shape[:-1] + (cols,), dtype=np.int8)
    bad = lib().or_unpack(_ptr(p, C.c_uint8), rows, cols, _ptr(out, C.c_int8))
    return out, int(bad)


def ternary_gemv(packed, cols: int, scale, x) -> np.ndarray:
    """y_r = scale_r * sum_i T[r][i] x_i (double) for a packed [rows][ceil(cols/4)] matrix."""
    p = _np(packed, np.uint8)
    rows = p.shape[0]
    assert p.shape == (rows, (cols + 3) // 4)
    sc = _np(scale, np.float64).reshape(rows)
    xv = _np(x, np.float64).reshape(cols)
    y = np.empty(rows, np.float64)
    lib().or_ternary_gemv(_ptr(p, C.c_uint8), rows, cols, _ptr(sc, C.c_double),
                          _ptr(xv, C.c_double), _ptr(y, C.c_double))
    _check_codes()
    return y


def pack3(w, row_bytes: int | None = None) -> tuple[np.ndarray, int]:
    """int8 [..., cols] -> base-3 packed uint8 [..., row_bytes] (five weights per byte, tw_oracle.h;
    row_bytes defaults to ceil(cols/5)), number of values outside {-1,0,1}."""
    w = _np(w, np.int8)
    cols = w.shape[-1]
    rb = (cols + 4) // 5 if row_bytes is None else int(row_bytes)
    assert rb >= (cols + 4) // 5
    rows = int(np.prod(w.shape[:-1])) if w.ndim > 1 else 1
    out = np.empty(w.shape[:-1] + (rb,), dtype=np.uint8)
    bad = lib().or_pack3(_ptr(w, C.c_int8), rows, cols, rb, _ptr(out, C.c_uint8))
    return out, int(bad)


def unpack3(packed, cols: int) -> tuple[np.ndarray, int]:
    """base-3 packed uint8 [..., row_bytes] -> int8 [..., cols], number of bytes above 242 met."""
    p = _np(packed, np.uint8)
    rb = p.shape[-1]
    assert rb >= (cols + 4) // 5
    rows = int(np.prod(p.shape[:-1])) if p.ndim > 1 else 1
    out = np.empty(p.shape[:-1] + (cols,), dtype=np.int8)
    bad = lib().or_unpack3(_ptr(p, C.c_uint8), rows, cols, rb, _ptr(out, C.c_int8))
    return out, int(bad)


def gemv_i8(w, scale, q, sx) -> np.ndarray:
    """int8 spec of y = s * (W q) on unpacked weights W [rows][cols] in {-1,0,1}: exact integer sum,
    then (float(sum) * sx) * s_r in fp32 (tw_oracle.h)."""
    wv = _np(w, np.int8)
    rows, cols = wv.shape
    sc = _np(scale, np.float32).reshape(rows)
    qv = _np(q, np.int8).reshape(cols)
    y = np.empty(rows, np.float32)
    lib().or_gemv_i8(_ptr(wv, C.c_int8), _ptr(sc, C.c_float), rows, cols, _ptr(qv, C.c_int8),
                     float(np.float32(sx)), _ptr(y, C.c_float))
    return y


def attention_decode(q, k, v) -> np.ndarray:
    """q [H][dh], k and v [n][Hkv][dh] (exact values widened to double) -> out [H][dh] (double):
    softmax(q_h . k_t / sqrt(dh)) weighted sum of v_t over the n cached positions, query head h
    reading KV head h / (H / Hkv) (tw_oracle.h)."""
    qv, kv, vv = _np(q, np.float64), _np(k, np.float64), _np(v, np.float64)
    H, dh = qv.shape
    n, Hkv, dh2 = kv.shape
    assert dh2 == dh and vv.shape == kv.shape and H % Hkv == 0
    out = np.empty((H, dh), np.float64)
    lib().or_attention_decode(_ptr(qv, C.c_double), _ptr(kv, C.c_double), _ptr(vv, C.c_double), n,
                              H, Hkv, dh, _ptr(out, C.c_double))
    return out


def flash_head(h, centroids, c_scale, wc, member_ids, top: int):
    """Approximate output head (tw_oracle.h): h [d] (fp32 values), centroids [ncl][d/2] u8 (offset
    nibbles), c_scale [ncl] fp32, wc [ncl][cs][d] (exact values, widened to double), member_ids
    [ncl][cs] int32 -> (sel [top] int32, ids [top][cs] int32, logits [top][cs] double, scores
    [ncl] fp32)."""
    hv = _np(h, np.float32).reshape(-1)
    d = hv.size
    cv = _np(centroids, np.uint8)
    ncl = cv.shape[0]
    assert cv.shape == (ncl, d // 2)
    sv = _np(c_scale, np.float32).reshape(ncl)
    wv = _np(wc, np.float64)
    cs = wv.shape[1]
    assert wv.shape == (ncl, cs, d)
    mv = _np(member_ids, np.int32).reshape(ncl, cs)
    sel = np.empty(top, np.int32)
    ids = np.empty((top, cs), np.int32)
    lg = np.empty((top, cs), np.float64)
    scores = np.empty(ncl, np.float32)
    lib().or_flash_head(_ptr(hv, C.c_float), d, _ptr(cv, C.c_uint8), _ptr(sv, C.c_float), ncl,
                        _ptr(wv, C.c_double), _ptr(mv, C.c_int32), cs, top, _ptr(sel, C.c_int32),
                        _ptr(ids, C.c_int32), _ptr(lg, C.c_double), _ptr(scores, C.c_float))
    return sel, ids, lg, scores


def round_bf16_bits(v) -> np.ndarray:
    v = _np(v, np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().or_round_bf16_array(_ptr(v, C.c_double), v.size, _ptr(out, C.c_uint16))
    return out


def bf16_bits_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def round_bf16(v) -> np.ndarray:
    """One round-to-nearest-even of doubles to bf16, returned as the (exact) float64 values."""
    return bf16_bits_to_f64(round_bf16_bits(v))


def round_f32(v) -> np.ndarray:
    v = _np(v, np.float64)
    out = np.empty(v.shape, dtype=np.float32)
    lib().or_round_f32_array(_ptr(v, C.c_double), v.size, _ptr(out, C.c_float))
    return out


def spec_expf(z) -> np.ndarray:
    z = _np(z, np.float32).ravel()
    f = lib().or_spec_expf
    return np.array([f(float(v)) for v in z], dtype=np.float32)


def quant_absmax(v) -> tuple[np.ndarray, np.float32]:
    v = _np(v, np.float32)
    q = np.empty(v.shape, dtype=np.int8)
    s = np.zeros(1, dtype=np.float32)
    lib().or_quant_absmax(_ptr(v, C.c_float), v.size, _ptr(q, C.c_int8), _ptr(s, C.c_float))
    return q, s[0]


# ---- layers ------------------------------------------------------------------------------------

class Layer:
    """One MoE FFN layer as the oracle sees it: router and scales as exact doubles, the ternary
    weights packed by the oracle's own ``pack``.

    ``t_gate``/``t_up`` are int8 [E][F][d], ``t_down`` int8 [E][d][F] with values in {-1,0,1};
    alternatively pass already-packed arrays with ``packed=True``."""

    def __init__(self, w_router, t_gate, t_up, t_down, s_gate, s_up, s_down,
                 pre_rmsnorm: bool = False, top_k: int = 8, packed: bool = False):
        self.w_router = _np(w_router, np.float64)
        E, d = self.w_router.shape
        if packed:
            self.p_gate = _np(t_gate, np.uint8)
            self.p_up = _np(t_up, np.uint8)
            self.p_down = _np(t_down, np.uint8)
            F = self.p_gate.shape[1]
        else:
            F = t_gate.shape[1]
            self.p_gate, b1 = pack(t_gate)
            self.p_up, b2 = pack(t_up)
            self.p_down, b3 = pack(t_down)
            if b1 or b2 or b3:
                raise ValueError("ternary weights hold values outside {-1,0,1}")
        self.s_gate = _np(s_gate, np.float64)
        self.s_up = _np(s_up, np.float64)
        self.s_down = _np(s_down, np.float64)
        self.s_gate32 = _np(s_gate, np.float32)
        self.s_up32 = _np(s_up, np.float32)
        self.s_down32 = _np(s_down, np.float32)
        self.d, self.F, self.E, self.k = d, F, E, int(top_k)
        self.pre_rmsnorm = bool(pre_rmsnorm)
        assert self.p_gate.shape == (E, F, (d + 3) // 4)
        assert self.p_up.shape == (E, F, (d + 3) // 4)
        assert self.p_down.shape == (E, d, (F + 3) // 4)
        assert self.s_gate.shape == (E, F) and self.s_up.shape == (E, F)
        assert self.s_down.shape == (E, d)
        self.c = _Layer(d, F, E, self.k, int(self.pre_rmsnorm), _ptr(self.w_router, C.c_double),
                        _ptr(self.p_gate, C.c_uint8), _ptr(self.p_up, C.c_uint8),
                        _ptr(self.p_down, C.c_uint8), _ptr(self.s_gate, C.c_double),
                        _ptr(self.s_up, C.c_double), _ptr(self.s_down, C.c_double))
        self.c8 = _LayerI8(d, F, E, self.k, _ptr(self.p_gate, C.c_uint8), _ptr(self.p_up, C.c_uint8),
                           _ptr(self.p_down, C.c_uint8), _ptr(self.s_gate32, C.c_float),
                           _ptr(self.s_up32, C.c_float), _ptr(self.s_down32, C.c_float))


def route(layer: Layer, x, n_threads: int = 1):
    """ids [T][k] int32, gates [T][k] float64, logits [T][E] float64 of the FFN input."""
    x = _np(x, np.float64).reshape(-1, layer.d)
    T = x.shape[0]
    ids = np.empty((T, layer.k), np.int32)
    g = np.empty((T, layer.k), np.float64)
    lg = np.empty((T, layer.E), np.float64)
    lib().or_route(C.byref(layer.c), _ptr(x, C.c_double), T, _ptr(ids, C.c_int32),
                   _ptr(g, C.c_double), _ptr(lg, C.c_double), n_threads)
    return ids, g, lg


def moe_layer(layer: Layer, x, n_threads: int = 1):
    """Route + FFN in double: out [T][d] (unrounded), ids, gates, logits."""
    x = _np(x, np.float64).reshape(-1, layer.d)
    T = x.shape[0]
    out = np.empty_like(x)
    ids = np.empty((T, layer.k), np.int32)
    g = np.empty((T, layer.k), np.float64)
    lg = np.empty((T, layer.E), np.float64)
    lib().or_moe_layer(C.byref(layer.c), _ptr(x, C.c_double), T, _ptr(out, C.c_double),
                       _ptr(ids, C.c_int32), _ptr(g, C.c_double), _ptr(lg, C.c_double), n_threads)
    _check_codes()
    return out, ids, g, lg


def ffn_token(layer: Layer, x, ids, gates, dense: bool = False):
    """out = x + sum_j g_j y_{ids_j} for one token under the given routing (double)."""
    x = _np(x, np.float64).reshape(layer.d)
    ids = _np(ids, np.int32).reshape(layer.k)
    gates = _np(gates, np.float64).reshape(layer.k)
    out = np.empty(layer.d, np.float64)
    f = lib().or_dense_ffn_token if dense else lib().or_ffn_token
    f(C.byref(layer.c), _ptr(x, C.c_double), _ptr(ids, C.c_int32), _ptr(gates, C.c_double),
      _ptr(out, C.c_double))
    _check_codes()
    return out


def decode_stack(layers: list[Layer], x0, n_steps: int):
    """Chained batch-1 decode.  Returns (layer_inputs [S][L][d], out [S][d], ids [S][L][k],
    gates [S][L][k], logits [S][L][E]); every value is bf16-exact."""
    arr = (_Layer * len(layers))(*[l.c for l in layers])
    d, k, E, nl = layers[0].d, layers[0].k, layers[0].E, len(layers)
    x0 = _np(x0, np.float64).reshape(d)
    li = np.empty((n_steps, nl, d), np.float64)
    out = np.empty((n_steps, d), np.float64)
    ids = np.empty((n_steps, nl, k), np.int32)
    g = np.empty((n_steps, nl, k), np.float64)
    lg = np.empty((n_steps, nl, E), np.float64)
    lib().or_decode_stack(arr, nl, _ptr(x0, C.c_double), n_steps, _ptr(li, C.c_double),
                          _ptr(out, C.c_double), _ptr(ids, C.c_int32), _ptr(g, C.c_double),
                          _ptr(lg, C.c_double))
    _check_codes()
    return li, out, ids, g, lg


def ffn_token_i8(layer: Layer, x, ids, gates):
    """int8 spec mode for one token; returns (out fp32 [d], taps dict)."""
    d, F, k = layer.d, layer.F, layer.k
    x = _np(x, np.float32).reshape(d)
    ids = _np(ids, np.int32).reshape(k)
    gates = _np(gates, np.float32).reshape(k)
    out = np.empty(d, np.float32)
    taps = dict(qx=np.empty(d, np.int8), sx=np.empty(1, np.float32),
                acc_gate=np.empty((k, F), np.int32), acc_up=np.empty((k, F), np.int32),
                qh=np.empty((k, F), np.int8), sh=np.empty(k, np.float32),
                acc_down=np.empty((k, d), np.int32), y=np.empty((k, d), np.float32))
    lib().or_ffn_token_i8(C.byref(layer.c8), _ptr(x, C.c_float), _ptr(ids, C.c_int32),
                          _ptr(gates, C.c_float), _ptr(out, C.c_float),
                          _ptr(taps["qx"], C.c_int8), _ptr(taps["sx"], C.c_float),
                          _ptr(taps["acc_gate"], C.c_int32), _ptr(taps["acc_up"], C.c_int32),
                          _ptr(taps["qh"], C.c_int8), _ptr(taps["sh"], C.c_float),
                          _ptr(taps["acc_down"], C.c_int32), _ptr(taps["y"], C.c_float))
    _check_codes()
    return out, taps


def ffn_batch_i8(layer: Layer, x, ids, gates, n_threads: int = 1):
    """int8 spec mode for T tokens under the given routing; out fp32 [T][d]."""
    x = _np(x, np.float32).reshape(-1, layer.d)
    T = x.shape[0]
    ids = _np(ids, np.int32).reshape(T, layer.k)
    gates = _np(gates, np.float32).reshape(T, layer.k)
    out = np.empty((T, layer.d), np.float32)
    lib().or_ffn_batch_i8(C.byref(layer.c8), _ptr(x, C.c_float), T, _ptr(ids, C.c_int32),
                          _ptr(gates, C.c_float), _ptr(out, C.c_float), n_threads)
    _check_codes()
    return out
