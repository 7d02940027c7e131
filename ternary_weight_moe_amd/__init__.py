"""Python binding of libternary_moe.so: the decode-time ternary MoE FFN on MI355X (gfx950).

Thin argument marshalling over the C ABI declared in include/ternary_moe.h: every step of the
computation runs in the library's HIP kernels.  PyTorch provides device memory and the current
stream only.  If the library is not built, every call raises (there is no fallback path).
"""
from __future__ import annotations

import ctypes as C
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# TW_LIB_PATH: another build of the same sources (for instance with sanitized host code)
LIB_PATH = os.environ.get("TW_LIB_PATH") or os.path.join(_HERE, "libternary_moe.so")

TW_F32, TW_BF16 = 0, 1
ACT_FLOAT, ACT_INT8 = 0, 1
_DT = {torch.float32: TW_F32, torch.bfloat16: TW_BF16}

_lock = threading.Lock()
_lib = None


class TwError(RuntimeError):
    """A non-zero tw_status returned by the library."""

    def __init__(self, what: str, status: int, text: str):
        super().__init__("%s: %s (status %d)" % (what, text, status))
        self.status = status


class TwLayer(C.Structure):
    """Mirror of tw_moe_layer (include/ternary_moe.h)."""
    _fields_ = [("d_model", C.c_int32), ("d_ff", C.c_int32), ("n_experts", C.c_int32),
                ("top_k", C.c_int32), ("router_dtype", C.c_int32), ("pre_rmsnorm", C.c_int32),
                ("w_router", C.c_void_p), ("w_gate", C.c_void_p), ("w_up", C.c_void_p),
                ("w_down", C.c_void_p), ("s_gate", C.c_void_p), ("s_up", C.c_void_p),
                ("s_down", C.c_void_p)]


EXPORTS = ("tw_status_str", "ternary_pack", "ternary_quantize", "ternary_pack3_row_bytes",
           "ternary_pack3", "ternary_gemv_i8", "attention_decode_workspace_bytes",
           "attention_decode", "attention_decode_one_workspace_bytes", "attention_decode_one",
           "flash_head_workspace_bytes", "flash_head", "moe_route_topk",
           "ternary_moe_ffn_decode", "ternary_moe_ffn_decode_static",
           "ternary_moe_decode_workspace_bytes", "ternary_moe_decode_error_offset",
           "ternary_moe_ffn_batched",
           "ternary_moe_batched_workspace_bytes")


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError("libternary_moe.so is not built (python -m "
                                   "ternary_weight_moe_amd.build); there is no fallback path")
            L = C.CDLL(LIB_PATH)
            i32, i64, vp, sz = C.c_int32, C.c_int64, C.c_void_p, C.c_size_t
            LP = C.POINTER(TwLayer)
            sig = {
                "tw_status_str": (C.c_char_p, [i32]),
                "ternary_pack": (i32, [vp, i64, i64, vp, vp, vp]),
                "ternary_quantize": (i32, [vp, i32, i64, i64, vp, vp, vp]),
                "ternary_pack3_row_bytes": (i64, [i64]),
                "ternary_pack3": (i32, [vp, i64, i64, vp, vp, vp]),
                "ternary_gemv_i8": (i32, [vp, i32, vp, i64, i64, vp, vp, vp, vp]),
                "attention_decode_workspace_bytes": (sz, [i32, i32, i64]),
                "attention_decode": (i32, [vp, vp, vp, i64, i32, i32, i32, vp, vp, sz, vp]),
                "attention_decode_one_workspace_bytes": (sz, [i32, i32, i64]),
                "attention_decode_one": (i32, [vp, vp, vp, i64, i32, i32, i32, vp, vp, sz, vp]),
                "flash_head_workspace_bytes": (sz, [i32]),
                "flash_head": (i32, [vp, i32, vp, vp, i32, vp, vp, i32, i32, vp, vp, vp, vp, sz,
                                     vp]),
                "moe_route_topk": (i32, [vp, i32, vp, i32, i64, i32, i32, i32, i32, vp, vp, vp,
                                         vp]),
                "ternary_moe_ffn_decode": (i32, [LP, i32, vp, vp, i32, vp, sz, vp]),
                "ternary_moe_ffn_decode_static": (i32, [LP, i32, vp, vp, i32, vp, vp]),
                "ternary_moe_decode_workspace_bytes": (sz, [LP, i32]),
                "ternary_moe_decode_error_offset": (sz, [LP, i32]),
                "ternary_moe_ffn_batched": (i32, [LP, i64, vp, i32, vp, i32, i32, vp, vp, vp, sz,
                                                  vp]),
                "ternary_moe_batched_workspace_bytes": (sz, [LP, i64, i32]),
            }
            for name, (res, args) in sig.items():
                f = getattr(L, name)
                f.restype = res
                f.argtypes = args
            _lib = L
        return _lib


def _check(status: int, what: str):
    if status != 0:
        raise TwError(what, status, lib().tw_status_str(status).decode())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _need_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("expected contiguous CUDA tensors")


# ---- ternary_pack --------------------------------------------------------------------------------

def ternary_pack(w: torch.Tensor, bad_count: torch.Tensor | None = None, out=None,
                 stream=None) -> torch.Tensor:
    """int8 [..., cols] with values in {-1,0,1} -> packed uint8 [..., ceil(cols/4)]."""
    _need_cuda(w, bad_count, out)
    if w.dtype != torch.int8:
        raise ValueError("ternary_pack expects int8")
    cols = w.shape[-1]
    rows = w.numel() // cols if cols else 0
    if out is None:
        out = torch.empty(w.shape[:-1] + ((cols + 3) // 4,), dtype=torch.uint8, device=w.device)
    _check(lib().ternary_pack(_ptr(w), rows, cols, _ptr(out), _ptr(bad_count), _stream(stream)),
           "ternary_pack")
    return out


def ternary_pack3_row_bytes(cols: int) -> int:
    """Bytes per row of the base-3 layout (five weights per byte, rows 16-byte aligned)."""
    return int(lib().ternary_pack3_row_bytes(int(cols)))


def ternary_pack3(w: torch.Tensor, bad_count: torch.Tensor | None = None, out=None,
                  stream=None) -> torch.Tensor:
    """int8 [..., cols] with values in {-1,0,1} -> base-3 packed uint8
    [..., ternary_pack3_row_bytes(cols)]."""
    _need_cuda(w, bad_count, out)
    if w.dtype != torch.int8:
        raise ValueError("ternary_pack3 expects int8")
    cols = w.shape[-1]
    rows = w.numel() // cols if cols else 0
    if out is None:
        out = torch.empty(w.shape[:-1] + (ternary_pack3_row_bytes(cols),), dtype=torch.uint8,
                          device=w.device)
    _check(lib().ternary_pack3(_ptr(w), rows, cols, _ptr(out), _ptr(bad_count), _stream(stream)),
           "ternary_pack3")
    return out


def ternary_gemv_i8(codes: torch.Tensor, layout: int, scales: torch.Tensor, cols: int,
                    xq: torch.Tensor, x_scale: torch.Tensor, out=None, stream=None) -> torch.Tensor:
    """y = (float(W q) * x_scale) * scales for ternary rows packed by ternary_pack (layout 2) or
    ternary_pack3 (layout 3); codes [rows][row bytes], scales [rows] fp32, xq [cols] int8,
    x_scale one fp32 (device), y [rows] fp32."""
    _need_cuda(codes, scales, xq, x_scale, out)
    rows = codes.shape[0]
    if out is None:
        out = torch.empty(rows, dtype=torch.float32, device=codes.device)
    _check(lib().ternary_gemv_i8(_ptr(codes), int(layout), _ptr(scales), rows, int(cols), _ptr(xq),
                                 _ptr(x_scale), _ptr(out), _stream(stream)), "ternary_gemv_i8")
    return out


def attention_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, out=None,
                     workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """One query token over a KV cache: q [H][128] bf16, k_cache and v_cache [n][Hkv][128] bf16
    (the filled slots) -> out [H][128] fp32; softmax(q_h . k_t / sqrt(128)) weighted sum of v_t,
    query head h reading KV head h / (H / Hkv)."""
    _need_cuda(q, k_cache, v_cache, out, workspace)
    if q.dtype != torch.bfloat16 or k_cache.dtype != torch.bfloat16 or v_cache.dtype != torch.bfloat16:
        raise ValueError("attention_decode expects bf16 q, k_cache and v_cache")
    H, dh = q.shape
    n, Hkv, dh2 = k_cache.shape
    if dh2 != dh or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch")
    if out is None:
        out = torch.empty((H, dh), dtype=torch.float32, device=q.device)
    nbytes = attention_decode_workspace_bytes(H, dh, n)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _check(lib().attention_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), n, H, Hkv, dh, _ptr(out),
                                  _ptr(workspace), workspace.numel(), _stream(stream)),
           "attention_decode")
    return out


def attention_decode_one(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                         workspace: torch.Tensor, out=None, stream=None) -> torch.Tensor:
    """attention_decode in one launch (at most 1024 slots).  `workspace` must be zero-filled before
    its first call (attention_decode_one_workspace) and used by this call only; each call leaves it
    zero-filled."""
    _need_cuda(q, k_cache, v_cache, out, workspace)
    if q.dtype != torch.bfloat16 or k_cache.dtype != torch.bfloat16 or v_cache.dtype != torch.bfloat16:
        raise ValueError("attention_decode_one expects bf16 q, k_cache and v_cache")
    H, dh = q.shape
    n, Hkv, dh2 = k_cache.shape
    if dh2 != dh or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch")
    if out is None:
        out = torch.empty((H, dh), dtype=torch.float32, device=q.device)
    _check(lib().attention_decode_one(_ptr(q), _ptr(k_cache), _ptr(v_cache), n, H, Hkv, dh,
                                      _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream)),
           "attention_decode_one")
    return out


def attention_decode_one_workspace(n_heads: int, head_dim: int, n_slots: int, device="cuda"):
    """A zero-filled workspace for attention_decode_one calls of up to n_slots slots."""
    nbytes = int(lib().attention_decode_one_workspace_bytes(int(n_heads), int(head_dim), int(n_slots)))
    if nbytes == 0:
        raise ValueError("attention_decode_one: unsupported shape")
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def flash_head(h: torch.Tensor, centroids: torch.Tensor, centroid_scales: torch.Tensor,
               w_clustered: torch.Tensor, member_ids: torch.Tensor, top: int, workspace=None,
               stream=None):
    """Approximate output head: h [d] bf16, centroids [ncl][d/2] uint8 (offset nibbles),
    centroid_scales [ncl] fp32, w_clustered [ncl][cs][d] bf16, member_ids [ncl][cs] int32 ->
    (sel_clusters [top] int32, token_ids [top][cs] int32, logits [top][cs] fp32)."""
    _need_cuda(h, centroids, centroid_scales, w_clustered, member_ids, workspace)
    if h.dtype != torch.bfloat16 or w_clustered.dtype != torch.bfloat16:
        raise ValueError("flash_head expects bf16 h and w_clustered")
    d = h.numel()
    ncl, cs, d2 = w_clustered.shape
    if d2 != d or centroids.shape != (ncl, d // 2) or member_ids.shape != (ncl, cs):
        raise ValueError("shape mismatch")
    dev = h.device
    sel = torch.empty(top, dtype=torch.int32, device=dev)
    ids = torch.empty((top, cs), dtype=torch.int32, device=dev)
    logits = torch.empty((top, cs), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(int(lib().flash_head_workspace_bytes(ncl)), 1),
                                dtype=torch.uint8, device=dev)
    _check(lib().flash_head(_ptr(h), d, _ptr(centroids), _ptr(centroid_scales), ncl,
                            _ptr(w_clustered), _ptr(member_ids), cs, int(top), _ptr(sel), _ptr(ids),
                            _ptr(logits), _ptr(workspace), workspace.numel(), _stream(stream)),
           "flash_head")
    return sel, ids, logits


def attention_decode_workspace_bytes(n_heads: int, head_dim: int, n_slots: int) -> int:
    return int(lib().attention_decode_workspace_bytes(int(n_heads), int(head_dim), int(n_slots)))


def ternary_quantize(w: torch.Tensor, packed: torch.Tensor | None = None,
                     scales: torch.Tensor | None = None, stream=None):
    """float [..., cols] (fp32 or bf16, cols a multiple of 8) -> (packed uint8 [..., cols/4],
    fp32 scales [...]) by the per-row absmean rule."""
    _need_cuda(w, packed, scales)
    if w.dtype not in _DT:
        raise ValueError("ternary_quantize expects fp32 or bf16")
    cols = w.shape[-1]
    rows = w.numel() // cols if cols else 0
    if packed is None:
        packed = torch.empty(w.shape[:-1] + (cols // 4,), dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty(w.shape[:-1], dtype=torch.float32, device=w.device)
    _check(lib().ternary_quantize(_ptr(w), _DT[w.dtype], rows, cols, _ptr(packed), _ptr(scales),
                                  _stream(stream)), "ternary_quantize")
    return packed, scales


# ---- routing -------------------------------------------------------------------------------------

def moe_route_topk(x: torch.Tensor, w_router: torch.Tensor, top_k: int, pre_rmsnorm: bool = False,
                   stream=None):
    """Router logits [T][E] fp32, expert ids [T][k] int32 and gates [T][k] fp32."""
    _need_cuda(x, w_router)
    x2 = x.reshape(-1, x.shape[-1])
    T, d = x2.shape
    E = w_router.shape[0]
    logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    ids = torch.empty((T, top_k), dtype=torch.int32, device=x.device)
    gates = torch.empty((T, top_k), dtype=torch.float32, device=x.device)
    _check(lib().moe_route_topk(_ptr(x2), _DT[x.dtype], _ptr(w_router), _DT[w_router.dtype], T,
                                d, E, top_k, int(pre_rmsnorm), _ptr(logits), _ptr(ids),
                                _ptr(gates), _stream(stream)), "moe_route_topk")
    return logits, ids, gates


# ---- layers --------------------------------------------------------------------------------------

class MoELayer:
    """One layer's device tensors (packed ternary weights, fp32 scales, router) and its
    tw_moe_layer descriptor."""

    def __init__(self, w_router, p_gate, p_up, p_down, s_gate, s_up, s_down, top_k: int,
                 pre_rmsnorm: bool = False):
        _need_cuda(w_router, p_gate, p_up, p_down, s_gate, s_up, s_down)
        self.w_router, self.p_gate, self.p_up, self.p_down = w_router, p_gate, p_up, p_down
        self.s_gate, self.s_up, self.s_down = s_gate, s_up, s_down
        E, d = w_router.shape
        F = p_gate.shape[1]
        self.d, self.F, self.E, self.k = d, F, E, int(top_k)
        self.pre_rmsnorm = bool(pre_rmsnorm)
        self.c = TwLayer(d, F, E, self.k, _DT[w_router.dtype], int(pre_rmsnorm),
                         w_router.data_ptr(), p_gate.data_ptr(), p_up.data_ptr(),
                         p_down.data_ptr(), s_gate.data_ptr(), s_up.data_ptr(), s_down.data_ptr())

    @classmethod
    def from_ternary(cls, w_router, t_gate, t_up, t_down, s_gate, s_up, s_down, top_k: int,
                     pre_rmsnorm: bool = False, stream=None):
        """Packs int8 ternary weights with ternary_pack (on the device) and keeps the result."""
        dev = w_router.device
        bad = torch.zeros(1, dtype=torch.int32, device=dev)
        p = [ternary_pack(t.to(dev).contiguous(), bad, stream=stream) for t in (t_gate, t_up, t_down)]
        layer = cls(w_router.to(dev).contiguous(), p[0], p[1], p[2], s_gate.to(dev).contiguous(),
                    s_up.to(dev).contiguous(), s_down.to(dev).contiguous(), top_k, pre_rmsnorm)
        layer.bad_count = bad
        return layer


    @classmethod
    def from_float(cls, w_router, w_gate, w_up, w_down, top_k: int, pre_rmsnorm: bool = False,
                   stream=None):
        """Quantises float expert weights (gate/up [E][F][d], down [E][d][F]) with
        ternary_quantize (on the device) and keeps the packed codes and per-row scales."""
        dev = w_router.device
        q = [ternary_quantize(t.to(dev).contiguous(), stream=stream) for t in (w_gate, w_up, w_down)]
        return cls(w_router.to(dev).contiguous(), q[0][0], q[1][0], q[2][0], q[0][1], q[1][1],
                   q[2][1], top_k, pre_rmsnorm)


def decode_workspace_bytes(layers) -> int:
    arr = (TwLayer * len(layers))(*[l.c for l in layers])
    return int(lib().ternary_moe_decode_workspace_bytes(arr, len(layers)))


def decode_error_flag(layers, workspace: torch.Tensor) -> int:
    """The decode health word of `workspace` after a completed ternary_moe_ffn_decode call on it
    (synchronises the device): nonzero if a hand-off wait of the stacked decode ran out."""
    layers = list(layers)
    arr = (TwLayer * len(layers))(*[l.c for l in layers])
    off = int(lib().ternary_moe_decode_error_offset(arr, len(layers)))
    if off == 0:
        raise ValueError("layers rejected by the library")
    torch.cuda.synchronize(workspace.device)
    return int(workspace[off:off + 4].view(torch.int32).item())


def batched_workspace_bytes(layer: MoELayer, n_tokens: int, act: str = "float") -> int:
    return int(lib().ternary_moe_batched_workspace_bytes(C.byref(layer.c), n_tokens,
                                                         ACT_INT8 if act == "int8" else ACT_FLOAT))


def ternary_moe_ffn_decode(layers, x: torch.Tensor, out: torch.Tensor | None = None,
                           workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Batch-1 decode of x [d] (fp32 or bf16) through the given layers; returns out [d]."""
    layers = list(layers)
    _need_cuda(x, out, workspace)
    arr = (TwLayer * len(layers))(*[l.c for l in layers])
    if out is None:
        out = torch.empty_like(x)
    if workspace is None:
        workspace = torch.empty(decode_workspace_bytes(layers), dtype=torch.uint8, device=x.device)
    _check(lib().ternary_moe_ffn_decode(arr, len(layers), _ptr(x), _ptr(out), _DT[x.dtype],
                                        _ptr(workspace), workspace.numel(), _stream(stream)),
           "ternary_moe_ffn_decode")
    return out


STATIC_SCRATCH_BYTES = 2 << 20   # TW_STATIC_SCRATCH_BYTES of include/ternary_moe.h


def ternary_moe_ffn_decode_static(layers, x: torch.Tensor, out: torch.Tensor | None = None,
                                  health: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """ternary_moe_ffn_decode with the library's static per-device scratch as its workspace (the C
    call allocates nothing); health: optional int32 device tensor of one element that receives
    the health word.  Calls that overlap on one device race on the shared scratch."""
    layers = list(layers)
    _need_cuda(x, out, health)
    arr = (TwLayer * len(layers))(*[l.c for l in layers])
    if out is None:
        out = torch.empty_like(x)
    _check(lib().ternary_moe_ffn_decode_static(arr, len(layers), _ptr(x), _ptr(out), _DT[x.dtype],
                                               _ptr(health) if health is not None else None,
                                               _stream(stream)),
           "ternary_moe_ffn_decode_static")
    return out


def ternary_moe_ffn_batched(layer: MoELayer, x: torch.Tensor, act: str = "float",
                            out_dtype: torch.dtype | None = None, expert_ids=None, gate_w=None,
                            out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                            stream=None) -> torch.Tensor:
    """One layer for T tokens x [T][d]; act "float" or "int8"; optional routing passed in."""
    _need_cuda(x, expert_ids, gate_w, out, workspace)
    T = x.shape[0]
    out_dtype = x.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((T, x.shape[1]), dtype=out_dtype, device=x.device)
    a = ACT_INT8 if act == "int8" else ACT_FLOAT
    if workspace is None:
        workspace = torch.empty(max(1, batched_workspace_bytes(layer, T, act)), dtype=torch.uint8,
                                device=x.device)
    _check(lib().ternary_moe_ffn_batched(C.byref(layer.c), T, _ptr(x), _DT[x.dtype], _ptr(out),
                                         _DT[out.dtype], a, _ptr(expert_ids), _ptr(gate_w),
                                         _ptr(workspace), workspace.numel(), _stream(stream)),
           "ternary_moe_ffn_batched")
    return out
