"""C-ABI checks that need no GPU: the library loads, exports every function include/ternary_moe.h
declares, and rejects bad arguments on the host before any HIP call (fake, never-dereferenced
device addresses are used; no kernel is launched)."""
import ctypes as C
import os
import re

import pytest

import ternary_weight_moe_amd as tw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ternary_moe.h")

OK, E_NULL, E_SHAPE, E_DTYPE, E_WS, E_ALIAS, E_UNSUP, E_HIP = 0, -1, -2, -3, -4, -5, -6, -7

# Fake device addresses, 256-byte aligned and far apart (never dereferenced: every call below fails
# its host-side checks before any HIP call).
A = [0x10000000 * (i + 1) for i in range(16)]


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(tw.LIB_PATH):
        from ternary_weight_moe_amd import build
        build.build()
    return tw.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert set(names) == set(tw.EXPORTS), names
    for n in names:
        assert hasattr(L, n)


def test_status_strings(L):
    for s in (OK, E_NULL, E_SHAPE, E_DTYPE, E_WS, E_ALIAS, E_UNSUP, E_HIP):
        assert L.tw_status_str(s) and L.tw_status_str(s) != b"unknown status"
    assert L.tw_status_str(12345) == b"unknown status"


def layer(d=2048, F=512, E=256, k=8, rdt=1, pre=0, base=0):
    return tw.TwLayer(d, F, E, k, rdt, pre, A[base], A[base + 1], A[base + 2], A[base + 3],
                      A[base + 4], A[base + 5], A[base + 6])


def test_pack_errors(L):
    s = C.c_void_p(0)
    assert L.ternary_pack(A[0], -1, 4, A[1], None, s) == E_SHAPE
    assert L.ternary_pack(A[0], 4, -1, A[1], None, s) == E_SHAPE
    assert L.ternary_pack(None, 4, 4, A[1], None, s) == E_NULL
    assert L.ternary_pack(A[0], 4, 4, None, None, s) == E_NULL
    assert L.ternary_pack(None, 0, 4, None, None, s) == OK        # empty: no-op
    assert L.ternary_pack(A[0], 4, 64, A[0] + 16, None, s) == E_ALIAS
    assert L.ternary_pack(A[0], 4, 64, A[1], A[1] + 4, s) == E_ALIAS


def test_route_errors(L):
    s = C.c_void_p(0)
    args = lambda **kw: [kw.get("x", A[0]), kw.get("xdt", 1), kw.get("w", A[1]), kw.get("wdt", 1),
                         kw.get("T", 4), kw.get("d", 2048), kw.get("E", 256), kw.get("k", 8),
                         kw.get("pre", 0), kw.get("lg", A[2]), kw.get("ids", A[3]),
                         kw.get("g", A[4]), s]
    assert L.moe_route_topk(*args(T=-1)) == E_SHAPE
    assert L.moe_route_topk(*args(k=0)) == E_SHAPE
    assert L.moe_route_topk(*args(k=9, E=8)) == E_SHAPE            # k > E
    assert L.moe_route_topk(*args(k=33, E=64)) == E_UNSUP          # k above 32
    assert L.moe_route_topk(*args(d=1000)) == E_UNSUP              # not a power of two
    assert L.moe_route_topk(*args(d=8192)) == E_UNSUP
    assert L.moe_route_topk(*args(E=2048)) == E_UNSUP
    assert L.moe_route_topk(*args(xdt=7)) == E_DTYPE
    assert L.moe_route_topk(*args(wdt=-1)) == E_DTYPE
    assert L.moe_route_topk(*args(pre=3)) == E_SHAPE
    assert L.moe_route_topk(*args(x=None)) == E_NULL
    assert L.moe_route_topk(*args(lg=None)) == E_NULL
    assert L.moe_route_topk(*args(ids=A[2] + 8)) == E_ALIAS        # ids inside logits
    assert L.moe_route_topk(*args(T=0, x=None)) == OK              # empty: no-op


def test_decode_errors(L):
    s = C.c_void_p(0)
    one = (tw.TwLayer * 1)(layer())
    need = L.ternary_moe_decode_workspace_bytes(one, 1)
    assert need > 0
    call = lambda ls, n=1, xi=A[8], xo=A[9], dt=1, ws=A[10], wsb=need: L.ternary_moe_ffn_decode(
        ls, n, xi, xo, dt, ws, wsb, s)
    assert call(None) == E_NULL
    assert call(one, n=0) == E_SHAPE
    assert call(one, n=65) == E_UNSUP
    assert call(one, xi=None) == E_NULL
    assert call(one, ws=None) == E_NULL
    assert call(one, dt=5) == E_DTYPE
    assert call(one, wsb=need - 1) == E_WS
    assert call(one, xo=A[8] + 2) == E_ALIAS
    assert call(one, ws=A[8] - 256, wsb=need + 4096) == E_ALIAS      # workspace over x_in
    bad = (tw.TwLayer * 1)(layer(d=1000))
    assert call(bad) == E_UNSUP
    bad = (tw.TwLayer * 1)(layer(k=300))
    assert call(bad) == E_SHAPE
    bad = (tw.TwLayer * 1)(layer(rdt=9))
    assert call(bad) == E_DTYPE
    l0 = layer()
    l0.w_up = None
    assert call((tw.TwLayer * 1)(l0)) == E_NULL
    l0 = layer()
    l0.w_down = A[3] + 8                                             # packed rows need 16-B alignment
    assert call((tw.TwLayer * 1)(l0)) == E_UNSUP
    l0 = layer()
    l0.s_up = A[5] + 4                                               # scales need 16-B alignment
    assert call((tw.TwLayer * 1)(l0)) == E_UNSUP
    assert call(one, ws=A[10] + 16) == E_UNSUP                       # workspace needs 256-B alignment
    two = (tw.TwLayer * 2)(layer(), layer(F=256))
    assert call(two, n=2) == E_SHAPE                                  # layers must match
    two = (tw.TwLayer * 2)(layer(), layer(pre=1))
    assert call(two, n=2) == E_SHAPE


def test_batched_errors(L):
    s = C.c_void_p(0)
    l = layer()
    need = L.ternary_moe_batched_workspace_bytes(C.byref(l), 64, 0)
    need8 = L.ternary_moe_batched_workspace_bytes(C.byref(l), 64, 1)
    assert need > 0 and need8 > 0
    assert L.ternary_moe_batched_workspace_bytes(C.byref(l), 64, 7) == 0
    call = lambda T=64, xi=A[8], idt=1, xo=A[9], odt=1, act=0, ids=None, g=None, ws=A[10], wsb=need, ll=None: \
        L.ternary_moe_ffn_batched(C.byref(ll if ll is not None else l), T, xi, idt, xo, odt, act,
                                  ids, g, ws, wsb, s)
    assert call(T=-1) == E_SHAPE
    assert call(idt=3) == E_DTYPE
    assert call(act=2) == E_DTYPE
    assert call(ids=A[11]) == E_NULL                                  # ids without gates
    assert call(xi=None) == E_NULL
    assert call(wsb=need - 1) == E_WS
    assert call(act=1, wsb=need8 - 1) == E_WS
    assert call(xo=A[8] + 64) == E_ALIAS
    assert call(T=0, xi=None, xo=None, ws=None) == OK
    assert call(act=1, ll=layer(pre=1), wsb=need8) == E_UNSUP         # int8 with pre-norm
    assert call(ws=A[10] + 128) == E_UNSUP                            # workspace needs 256-B alignment
    assert call(xi=A[8] + 8) == E_UNSUP                               # activations need 16-B alignment
    assert L.ternary_moe_ffn_batched(None, 4, A[8], 1, A[9], 1, 0, None, None, A[10], need, s) == E_NULL


def test_quantize_errors(L):
    s = None
    F32, BF16 = 0, 1
    assert L.ternary_quantize(A[0], BF16, -1, 64, A[1], A[2], s) == E_SHAPE
    assert L.ternary_quantize(A[0], BF16, 4, -8, A[1], A[2], s) == E_SHAPE
    assert L.ternary_quantize(A[0], 7, 4, 64, A[1], A[2], s) == E_DTYPE
    assert L.ternary_quantize(None, BF16, 0, 64, None, None, s) == OK       # empty: no-op
    assert L.ternary_quantize(None, BF16, 4, 64, A[1], A[2], s) == E_NULL
    assert L.ternary_quantize(A[0], BF16, 4, 64, None, A[2], s) == E_NULL
    assert L.ternary_quantize(A[0], BF16, 4, 64, A[1], None, s) == E_NULL
    assert L.ternary_quantize(A[0], F32, 4, 12, A[1], A[2], s) == E_UNSUP    # cols % 8
    assert L.ternary_quantize(A[0], F32, 4, 65544, A[1], A[2], s) == E_UNSUP
    assert L.ternary_quantize(A[0] + 8, F32, 4, 64, A[1], A[2], s) == E_UNSUP
    assert L.ternary_quantize(A[0], F32, 4, 64, A[1] + 8, A[2], s) == E_UNSUP
    assert L.ternary_quantize(A[0], F32, 4, 64, A[1], A[2] + 2, s) == E_UNSUP
    assert L.ternary_quantize(A[0], F32, 4, 64, A[0] + 512, A[2], s) == E_ALIAS   # inside w
    assert L.ternary_quantize(A[0], F32, 4, 64, A[1], A[0] + 16, s) == E_ALIAS
    assert L.ternary_quantize(A[0], F32, 4, 64, A[1], A[1] + 32, s) == E_ALIAS    # inside packed


def test_decode_error_offset_inside_the_workspace(L):
    lay = layer()
    n = L.ternary_moe_decode_workspace_bytes(C.byref(lay), 1)
    off = L.ternary_moe_decode_error_offset(C.byref(lay), 1)
    assert 0 < off and off + 4 <= n and off % 4 == 0
    assert L.ternary_moe_decode_error_offset(None, 1) == 0
    assert L.ternary_moe_decode_error_offset(C.byref(layer(k=0)), 1) == 0


def test_pack3_row_bytes_and_errors(L):
    assert [L.ternary_pack3_row_bytes(c) for c in (0, 1, 5, 80, 81, 2048, 512, 5120)] == \
        [0, 16, 16, 16, 32, 416, 112, 1024]
    assert L.ternary_pack3_row_bytes(-1) == -1
    s = C.c_void_p(0)
    assert L.ternary_pack3(A[0], -1, 5, A[1], None, s) == E_SHAPE
    assert L.ternary_pack3(A[0], 4, -1, A[1], None, s) == E_SHAPE
    assert L.ternary_pack3(None, 4, 5, A[1], None, s) == E_NULL
    assert L.ternary_pack3(A[0], 4, 5, None, None, s) == E_NULL
    assert L.ternary_pack3(None, 0, 5, None, None, s) == OK        # empty: no-op
    assert L.ternary_pack3(A[0], 4, 64, A[0] + 16, None, s) == E_ALIAS
    assert L.ternary_pack3(A[0], 4, 64, A[1], A[1] + 60, s) == E_ALIAS   # inside 4 x 16 bytes
    assert L.ternary_pack3(A[0], 4, 64, A[1], A[0] + 4, s) == E_ALIAS


def test_gemv_i8_errors(L):
    s = None
    g = L.ternary_gemv_i8
    assert g(A[0], 3, A[1], -1, 2048, A[2], A[3], A[4], s) == E_SHAPE
    assert g(A[0], 3, A[1], 4, -1, A[2], A[3], A[4], s) == E_SHAPE
    assert g(A[0], 4, A[1], 4, 2048, A[2], A[3], A[4], s) == E_DTYPE
    assert g(None, 3, None, 0, 2048, None, None, None, s) == OK     # empty: no-op
    for i in range(5):
        args = [A[0], A[1], A[2], A[3], A[4]]
        args[i] = None
        assert g(args[0], 3, args[1], 4, 2048, args[2], args[3], args[4], s) == E_NULL
    assert g(A[0], 2, A[1], 4, 2000, A[2], A[3], A[4], s) == E_UNSUP     # 2-bit: cols % 64
    assert g(A[0], 2, A[1], 4, 4160, A[2], A[3], A[4], s) == E_UNSUP     # 2-bit: above 4096
    assert g(A[0], 3, A[1], 4, 5125, A[2], A[3], A[4], s) == E_UNSUP     # base 3: above 5120
    assert g(A[0], 3, A[1], 4, 0, A[2], A[3], A[4], s) == E_UNSUP
    assert g(A[0] + 8, 3, A[1], 4, 2048, A[2], A[3], A[4], s) == E_UNSUP
    assert g(A[0], 3, A[1] + 2, 4, 2048, A[2], A[3], A[4], s) == E_UNSUP
    assert g(A[0], 3, A[1], 4, 2048, A[2], A[3] + 1, A[4], s) == E_UNSUP
    assert g(A[0], 3, A[1], 4, 2048, A[2], A[3], A[4] + 2, s) == E_UNSUP
    assert g(A[0], 3, A[1], 4, 2048, A[2], A[3], A[0] + 1600, s) == E_ALIAS   # inside codes
    assert g(A[0], 3, A[1], 4, 2048, A[2], A[3], A[1] + 8, s) == E_ALIAS
    assert g(A[0], 3, A[1], 4, 2048, A[2], A[3], A[2] + 2044, s) == E_ALIAS
    assert g(A[0], 3, A[1], 4, 2048, A[2], A[3], A[3] - 12, s) == E_ALIAS


def test_attention_decode_workspace_and_errors(L):
    ws = L.attention_decode_workspace_bytes
    assert ws(16, 128, 640) == ((640 + 15) // 16 * 16 * 130 * 4 + 255) // 256 * 256
    assert ws(16, 64, 640) == 0 and ws(0, 128, 640) == 0 and ws(16, 128, 0) == 0
    assert ws(16, 128, (1 << 21) + 1) == 0
    s = None
    a = L.attention_decode
    big = 1 << 30
    assert a(A[0], A[1], A[2], 0, 16, 4, 128, A[3], A[4], big, s) == E_SHAPE
    assert a(A[0], A[1], A[2], (1 << 21) + 1, 16, 4, 128, A[3], A[4], big, s) == E_SHAPE
    assert a(A[0], A[1], A[2], 640, 16, 3, 128, A[3], A[4], big, s) == E_SHAPE     # 16 % 3
    assert a(A[0], A[1], A[2], 640, 0, 1, 128, A[3], A[4], big, s) == E_SHAPE
    assert a(A[0], A[1], A[2], 640, 16, 4, 64, A[3], A[4], big, s) == E_UNSUP      # head_dim
    assert a(A[0], A[1], A[2], 640, 48, 3, 128, A[3], A[4], big, s) == E_UNSUP     # group 16
    assert a(A[0], A[1], A[2], 640, 12, 4, 128, A[3], A[4], big, s) == E_UNSUP     # group 3
    assert a(A[0], A[1], A[2], 640, 256, 32, 128, A[3], A[4], big, s) == E_UNSUP   # > 128 heads
    for i in range(5):
        args = [A[0], A[1], A[2], A[3], A[4]]
        args[i] = None
        assert a(args[0], args[1], args[2], 640, 16, 4, 128, args[3], args[4], big, s) == E_NULL
    assert a(A[0] + 8, A[1], A[2], 640, 16, 4, 128, A[3], A[4], big, s) == E_UNSUP
    assert a(A[0], A[1], A[2] + 8, 640, 16, 4, 128, A[3], A[4], big, s) == E_UNSUP
    assert a(A[0], A[1], A[2], 640, 16, 4, 128, A[3] + 2, A[4], big, s) == E_UNSUP
    assert a(A[0], A[1], A[2], 640, 16, 4, 128, A[3], A[4] + 16, big, s) == E_UNSUP
    assert a(A[0], A[1], A[2], 640, 16, 4, 128, A[3], A[4], ws(16, 128, 640) - 1, s) == E_WS
    assert a(A[0], A[1], A[2], 640, 16, 4, 128, A[1] + 4096, A[4], big, s) == E_ALIAS   # in k
    assert a(A[0], A[1], A[2], 640, 16, 4, 128, A[0], A[4], big, s) == E_ALIAS
    assert a(A[0], A[1], A[2], 640, 16, 4, 128, A[3], A[2] + 1024, big, s) == E_ALIAS   # ws in v
    assert a(A[0], A[1], A[2], 640, 16, 4, 128, A[4] + 512, A[4], big, s) == E_ALIAS    # out in ws


def test_attention_decode_one_workspace_and_errors(L):
    ws = L.attention_decode_one_workspace_bytes
    assert ws(16, 128, 640) == ((640 + 15) // 16 * 16 * 130 * 8 + 255) // 256 * 256
    assert ws(16, 128, 1024) > 0 and ws(16, 128, 1025) == 0      # at most 64 splits of 16
    assert ws(16, 64, 640) == 0 and ws(0, 128, 640) == 0 and ws(16, 128, 0) == 0
    s = None
    a = L.attention_decode_one
    big = 1 << 30
    assert a(A[0], A[1], A[2], 0, 16, 4, 128, A[3], A[4], big, s) == E_SHAPE
    assert a(A[0], A[1], A[2], 640, 16, 3, 128, A[3], A[4], big, s) == E_SHAPE
    assert a(A[0], A[1], A[2], 1025, 16, 4, 128, A[3], A[4], big, s) == E_UNSUP    # > 64 splits
    assert a(A[0], A[1], A[2], 640, 16, 4, 64, A[3], A[4], big, s) == E_UNSUP
    assert a(A[0], A[1], A[2], 640, 12, 4, 128, A[3], A[4], big, s) == E_UNSUP     # group 3
    for i in range(5):
        args = [A[0], A[1], A[2], A[3], A[4]]
        args[i] = None
        assert a(args[0], args[1], args[2], 640, 16, 4, 128, args[3], args[4], big, s) == E_NULL
    assert a(A[0] + 8, A[1], A[2], 640, 16, 4, 128, A[3], A[4], big, s) == E_UNSUP
    assert a(A[0], A[1], A[2], 640, 16, 4, 128, A[3], A[4] + 16, big, s) == E_UNSUP
    assert a(A[0], A[1], A[2], 640, 16, 4, 128, A[3], A[4], ws(16, 128, 640) - 1, s) == E_WS
    assert a(A[0], A[1], A[2], 640, 16, 4, 128, A[1] + 4096, A[4], big, s) == E_ALIAS   # in k
    assert a(A[0], A[1], A[2], 640, 16, 4, 128, A[3], A[2] + 1024, big, s) == E_ALIAS   # ws in v
    assert a(A[0], A[1], A[2], 640, 16, 4, 128, A[4] + 512, A[4], big, s) == E_ALIAS    # out in ws


def test_flash_head_workspace_and_errors(L):
    assert L.flash_head_workspace_bytes(4748) == (4748 * 4 + 255) // 256 * 256
    assert L.flash_head_workspace_bytes(0) == 0 and L.flash_head_workspace_bytes(8193) == 0
    f = L.flash_head
    big = 1 << 30
    ok = [A[0], 2048, A[1], A[2], 4748, A[15], A[4], 32, 512, A[5], A[6], A[7], A[8], big, None]

    def call(**kw):
        a = list(ok)
        names = ["h", "d", "cent", "cs_", "ncl", "w", "mem", "csz", "top", "sel", "ids", "lg", "ws",
                 "wsb", "s"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return f(*a)
    assert call(ncl=0) == E_SHAPE and call(ncl=8193) == E_SHAPE
    assert call(csz=0) == E_SHAPE and call(csz=1025) == E_SHAPE
    assert call(top=0) == E_SHAPE and call(top=4749) == E_SHAPE
    assert call(d=0) == E_SHAPE
    assert call(d=1536) == E_UNSUP and call(d=8192) == E_UNSUP
    for k in ["h", "cent", "cs_", "w", "mem", "sel", "ids", "lg", "ws"]:
        assert call(**{k: None}) == E_NULL, k
    assert call(cent=A[1] + 8) == E_UNSUP and call(w=A[15] + 8) == E_UNSUP
    assert call(h=A[0] + 1) == E_UNSUP and call(lg=A[7] + 2) == E_UNSUP and call(ws=A[8] + 64) == E_UNSUP
    assert call(wsb=L.flash_head_workspace_bytes(4748) - 1) == E_WS
    assert call(lg=A[15] + 4096) == E_ALIAS       # logits inside the head rows
    assert call(ids=A[7] + 4) == E_ALIAS          # ids overlapping logits
    assert call(ws=A[5]) == E_ALIAS               # workspace over sel


def test_decode_static_errors(L):
    s = C.c_void_p(0)
    one = (tw.TwLayer * 1)(layer())
    # the same argument checks as ternary_moe_ffn_decode (no workspace argument)
    assert L.ternary_moe_ffn_decode_static(None, 1, A[8], A[9], 1, None, s) == E_NULL
    assert L.ternary_moe_ffn_decode_static(one, 0, A[8], A[9], 1, None, s) == E_SHAPE
    assert L.ternary_moe_ffn_decode_static(one, 1, None, A[9], 1, None, s) == E_NULL
    assert L.ternary_moe_ffn_decode_static(one, 1, A[8], A[8] + 64, 1, None, s) == E_ALIAS
    assert L.ternary_moe_ffn_decode_static(one, 1, A[8], A[9], 7, None, s) == E_DTYPE
    # the health word: 4-byte aligned, not overlapping the activations
    assert L.ternary_moe_ffn_decode_static(one, 1, A[8], A[9], 1, A[10] + 2, s) == E_UNSUP
    assert L.ternary_moe_ffn_decode_static(one, 1, A[8], A[9], 1, A[9] + 8, s) == E_ALIAS
    # layers whose workspace exceeds the static scratch are rejected before any HIP call
    big = (tw.TwLayer * 1)(layer(d=4096, F=1024, E=1024, k=16))
    need = L.ternary_moe_decode_workspace_bytes(big, 1)
    assert need > tw.STATIC_SCRATCH_BYTES
    assert L.ternary_moe_ffn_decode_static(big, 1, A[8], A[9], 1, None, s) == E_WS
    # the full-size stack fits
    stack = (tw.TwLayer * 24)(*[layer() for _ in range(24)])
    assert L.ternary_moe_decode_workspace_bytes(stack, 24) <= tw.STATIC_SCRATCH_BYTES
