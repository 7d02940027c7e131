"""Pins for the CPU oracle: each check ties the oracle to something other than itself -- values the
pages print, closed forms, invariants, special cases that reduce to a library routine, or brute
force on tiny inputs -- so that a dropped term, a wrong sign or index, or a transposed operand in
the oracle fails at least one of them.  CPU only.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from ternary_weight_moe_amd import accounting

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(12345)


def rand_trits(*shape):
    return rng.integers(-1, 2, size=shape, dtype=np.int8)


def tiny_layer(d=16, F=8, E=4, k=2, pre=False, seed=0, router_std=0.3):
    r = np.random.default_rng(seed)
    w = dict(
        w_router=r.normal(0, router_std, (E, d)).astype(np.float32),
        t_gate=r.integers(-1, 2, (E, F, d), dtype=np.int8),
        t_up=r.integers(-1, 2, (E, F, d), dtype=np.int8),
        t_down=r.integers(-1, 2, (E, d, F), dtype=np.int8),
        s_gate=r.uniform(0.01, 0.1, (E, F)).astype(np.float32),
        s_up=r.uniform(0.01, 0.1, (E, F)).astype(np.float32),
        s_down=r.uniform(0.01, 0.1, (E, d)).astype(np.float32),
    )
    return w, oracle.Layer(**w, pre_rmsnorm=pre, top_k=k)


# ---- packing -----------------------------------------------------------------------------------

def test_pack_reading_single_weights():
    # Reading of the 2-bit code: 00 -> 0, 01 -> +1, 10 -> -1, weight j of a byte in bits 2j..2j+1.
    for j in range(4):
        for v, code in ((0, 0), (1, 1), (-1, 2)):
            w = np.zeros((1, 4), np.int8)
            w[0, j] = v
            p, bad = oracle.pack(w)
            assert bad == 0 and p[0, 0] == code << (2 * j)


def test_pack_exhaustive_81_patterns_bijective():
    pats = np.array(np.meshgrid(*[[-1, 0, 1]] * 4, indexing="ij")).reshape(4, -1).T.astype(np.int8)
    assert pats.shape == (81, 4)
    p, bad = oracle.pack(pats)
    assert bad == 0
    bytes_ = p[:, 0]
    assert len(set(bytes_.tolist())) == 81                      # injective
    assert all(((b >> (2 * j)) & 3) != 3 for b in bytes_ for j in range(4))   # never code 11
    back, bad = oracle.unpack(p, 4)
    assert bad == 0 and np.array_equal(back, pats)


def test_unpack_all_256_bytes_rejects_code_11():
    allb = np.arange(256, dtype=np.uint8).reshape(256, 1)
    w, bad = oracle.unpack(allb, 4)
    n11 = sum(1 for b in range(256) for j in range(4) if ((b >> (2 * j)) & 3) == 3)
    assert bad == n11
    assert 256 - sum(1 for b in range(256) if any(((b >> (2 * j)) & 3) == 3 for j in range(4))) == 81


def test_pack_round_trip_ragged_and_bad_values():
    for cols in (1, 3, 4, 5, 130, 2049):
        w = rand_trits(7, cols)
        p, bad = oracle.pack(w)
        assert bad == 0 and p.shape == (7, (cols + 3) // 4)
        back, bad = oracle.unpack(p, cols)
        assert bad == 0 and np.array_equal(back, w)
        # padding weights of the last byte are code 00
        if cols % 4:
            assert np.all((p[:, -1] >> (2 * (cols % 4))) == 0)
    w = rand_trits(3, 9)
    w[1, 4] = 2
    w[2, 0] = -5
    p, bad = oracle.pack(w)
    assert bad == 2


# ---- ternary GEMV ---------------------------------------------------------------------------------

def test_gemv_one_hot_reproduces_scaled_weight_columns():
    T = rand_trits(37, 53)
    s = rng.uniform(0.01, 0.1, 37)
    p, _ = oracle.pack(T)
    for k in (0, 1, 26, 52):
        x = np.zeros(53)
        x[k] = 1.0
        y = oracle.ternary_gemv(p, 53, s, x)
        assert np.array_equal(y, s * T[:, k])           # column k, scaled by row scales, exactly


def test_gemv_closed_forms():
    x = rng.normal(size=64)
    s = rng.uniform(0.01, 0.1, 5)
    ones = np.ones((5, 64), np.int8)
    y = oracle.ternary_gemv(oracle.pack(ones)[0], 64, s, x)
    assert np.allclose(y, s * x.sum(), rtol=1e-14)
    y = oracle.ternary_gemv(oracle.pack(-ones)[0], 64, s, x)
    assert np.allclose(y, -s * x.sum(), rtol=1e-14)
    y = oracle.ternary_gemv(oracle.pack(np.zeros((5, 64), np.int8))[0], 64, s, x)
    assert np.all(y == 0.0)
    # integer inputs: exact integer sums, equal to an int64 matmul of the unpacked matrix
    T = rand_trits(9, 301)
    xi = rng.integers(-1000, 1000, 301)
    y = oracle.ternary_gemv(oracle.pack(T)[0], 301, np.ones(9), xi.astype(np.float64))
    assert np.array_equal(y, (T.astype(np.int64) @ xi).astype(np.float64))


def test_gemv_matches_library_matmul():
    T = rand_trits(29, 77)
    s = rng.uniform(0.01, 0.1, 29)
    x = rng.normal(size=77)
    y = oracle.ternary_gemv(oracle.pack(T)[0], 77, s, x)
    ref = (torch.from_numpy(s)[:, None] * torch.from_numpy(T.astype(np.float64))) @ torch.from_numpy(x)
    assert np.allclose(y, ref.numpy(), rtol=1e-12, atol=1e-14)


# ---- routing ------------------------------------------------------------------------------------

def test_route_zero_input_ties_go_to_lower_ids():
    for k in (1, 2, 4):
        w, L = tiny_layer(k=k)
        ids, g, lg = oracle.route(L, np.zeros((1, 16)))
        assert np.all(lg == 0)
        assert ids[0].tolist() == list(range(k))
        assert np.allclose(g[0], 1.0 / k, rtol=0, atol=1e-15)


def test_route_matches_library_sort_and_softmax():
    w, L = tiny_layer(d=32, E=8, k=3)
    x = rng.normal(size=(20, 32)).astype(np.float32)
    ids, g, lg = oracle.route(L, x)
    ref_l = x.astype(np.float64) @ w["w_router"].astype(np.float64).T
    assert np.allclose(lg, ref_l, rtol=1e-12, atol=1e-12)
    for t in range(20):
        order = np.lexsort((np.arange(8), -ref_l[t]))[:3]       # descending logit, then lower id
        assert ids[t].tolist() == order.tolist()
        ref_g = torch.softmax(torch.from_numpy(ref_l[t, order]), 0).numpy()
        assert np.allclose(g[t], ref_g, rtol=1e-12)
        assert abs(g[t].sum() - 1.0) < 1e-14
        # ratio of two gates is the exponential of the logit gap
        assert math.isclose(g[t, 0] / g[t, 1], math.exp(ref_l[t, order[0]] - ref_l[t, order[1]]),
                            rel_tol=1e-12)


def test_route_k1_gate_is_one_and_k_equals_E():
    w, L = tiny_layer(k=1)
    ids, g, _ = oracle.route(L, rng.normal(size=(5, 16)))
    assert np.all(g == 1.0)
    w, L = tiny_layer(E=4, k=4)
    ids, g, lg = oracle.route(L, rng.normal(size=(5, 16)))
    assert all(sorted(r) == [0, 1, 2, 3] for r in ids.tolist())
    full = torch.softmax(torch.from_numpy(lg), 1).numpy()
    assert np.allclose(np.take_along_axis(full, ids, 1), g, rtol=1e-12)


def test_route_permuting_experts_permutes_ids():
    w, L = tiny_layer(d=24, E=8, k=3)
    perm = rng.permutation(8)
    w2 = dict(w)
    for key in ("w_router", "t_gate", "t_up", "t_down", "s_gate", "s_up", "s_down"):
        w2[key] = w[key][perm]
    L2 = oracle.Layer(**w2, top_k=3)
    x = rng.normal(size=(10, 24))
    ids1, g1, _ = oracle.route(L, x)
    ids2, g2, _ = oracle.route(L2, x)
    assert np.array_equal(perm[ids2], ids1)
    assert np.array_equal(g1, g2)
    out1, *_ = oracle.moe_layer(L, x)
    out2, *_ = oracle.moe_layer(L2, x)
    assert np.allclose(out1, out2, rtol=1e-13, atol=1e-13)


# ---- expert FFN -----------------------------------------------------------------------------------

def _torch_ffn(w, x, ids, g, pre=False):
    """Independent evaluation with torch fp64 library routines on the unpacked matrices."""
    xt = torch.from_numpy(np.asarray(x, np.float64))
    xn = xt / torch.sqrt((xt * xt).mean() + 1e-6) if pre else xt
    out = xt.clone()
    for j, e in enumerate(ids):
        Wg = torch.from_numpy(w["s_gate"][e].astype(np.float64))[:, None] * torch.from_numpy(w["t_gate"][e].astype(np.float64))
        Wu = torch.from_numpy(w["s_up"][e].astype(np.float64))[:, None] * torch.from_numpy(w["t_up"][e].astype(np.float64))
        Wd = torch.from_numpy(w["s_down"][e].astype(np.float64))[:, None] * torch.from_numpy(w["t_down"][e].astype(np.float64))
        h = torch.nn.functional.silu(Wg @ xn) * (Wu @ xn)
        out = out + float(g[j]) * (Wd @ h)
    return out.numpy()


@pytest.mark.parametrize("d,F,E,k,pre", [(8, 4, 4, 1, False), (16, 8, 4, 2, False),
                                         (64, 32, 8, 8, False), (64, 32, 8, 2, True),
                                         (21, 6, 5, 3, False)])
def test_ffn_matches_dense_brute_force_and_library(d, F, E, k, pre):
    w, L = tiny_layer(d=d, F=F, E=E, k=k, pre=pre, seed=d + F)
    x = rng.normal(size=(4, d)) * 3.0
    out, ids, g, _ = oracle.moe_layer(L, x)
    for t in range(4):
        dense = oracle.ffn_token(L, x[t], ids[t], g[t], dense=True)
        assert np.allclose(out[t], dense, rtol=1e-12, atol=1e-12)
        ref = _torch_ffn(w, x[t], ids[t], g[t], pre)
        assert np.allclose(out[t], ref, rtol=1e-11, atol=1e-12)


def test_ffn_all_zero_codes_is_identity_and_zero_input_is_zero():
    w, L = tiny_layer(d=32, F=16, E=4, k=2)
    z = dict(w, t_gate=np.zeros_like(w["t_gate"]), t_up=np.zeros_like(w["t_up"]),
             t_down=np.zeros_like(w["t_down"]))
    Lz = oracle.Layer(**z, top_k=2)
    x = rng.normal(size=(3, 32)).astype(np.float32).astype(np.float64)
    out, *_ = oracle.moe_layer(Lz, x)
    assert np.array_equal(out, x)
    for pre in (False, True):
        w2, L2 = tiny_layer(d=32, F=16, E=4, k=2, pre=pre)
        out, *_ = oracle.moe_layer(L2, np.zeros((1, 32)))
        assert np.all(out == 0.0)


def test_ffn_down_scale_power_of_two_scales_contribution_exactly():
    w, L = tiny_layer(d=32, F=16, E=4, k=2)
    x = rng.normal(size=(2, 32))
    out1, ids, g, _ = oracle.moe_layer(L, x)
    w8 = dict(w, s_down=w["s_down"] * 8)
    out8, ids8, g8, _ = oracle.moe_layer(oracle.Layer(**w8, top_k=2), x)
    assert np.array_equal(ids, ids8)
    # (x + c) - x recovers c up to one rounding of the residual add, i.e. half an ulp of out
    bound = 8 * np.spacing(np.maximum(np.abs(out8), np.abs(out1)))
    assert np.all(np.abs((out8 - x) - 8 * (out1 - x)) <= bound)
    # the ternary product itself scales exactly
    T = w["t_down"][0]
    h = rng.normal(size=16)
    y1 = oracle.ternary_gemv(oracle.pack(T)[0], 16, w["s_down"][0], h)
    y8 = oracle.ternary_gemv(oracle.pack(T)[0], 16, w["s_down"][0] * 8, h)
    assert np.array_equal(y8, 8 * y1)


def test_ffn_one_hot_input_closed_form():
    # With T_u = T_g and s_u = s_g, a one-hot input e_c gives gate_r = up_r = a_r = s_r * T[r][c],
    # so h_r = a_r^2 * sigmoid(a_r); with T_d = identity (F = d) and s_d = 1, y = h.
    d = F = 12
    E, k = 3, 1
    r = np.random.default_rng(3)
    Tg = r.integers(-1, 2, (E, F, d), dtype=np.int8)
    sg = r.uniform(0.5, 2.0, (E, F)).astype(np.float32)
    eye = np.broadcast_to(np.eye(d, dtype=np.int8), (E, d, F)).copy()
    L = oracle.Layer(np.zeros((E, d), np.float32), Tg, Tg, eye, sg, sg, np.ones((E, d), np.float32),
                     top_k=k)
    for c in (0, 5, 11):
        x = np.zeros(d)
        x[c] = 1.0
        out = oracle.ffn_token(L, x, [2], [1.0])
        a = sg[2].astype(np.float64) * Tg[2, :, c]
        expect = x + a * a / (1.0 + np.exp(-a))
        assert np.allclose(out, expect, rtol=1e-15, atol=1e-16)


def test_pre_rmsnorm_properties():
    # x with mean(x^2) = 1: the FFN input is x / sqrt(1 + 1e-6); logits of c*x equal those of x
    # up to the epsilon; the residual is not normalised.
    w, L = tiny_layer(d=64, F=16, E=8, k=2, pre=True)
    x = rng.choice([-1.0, 1.0], size=(1, 64))
    _, _, lg = oracle.route(L, x)
    assert np.allclose(lg[0], (w["w_router"].astype(np.float64) @ x[0]) / math.sqrt(1 + 1e-6),
                       rtol=1e-14)
    _, _, lg4 = oracle.route(L, 4 * x)
    assert np.allclose(lg4, lg, rtol=1e-6)
    out1, *_ = oracle.moe_layer(L, x)
    out4, *_ = oracle.moe_layer(L, 4 * x)
    c1, c4 = out1 - x, out4 - 4 * x
    assert np.max(np.abs(c4 - c1)) <= 1e-5 * np.max(np.abs(c1))


def test_batched_equals_per_token():
    w, L = tiny_layer(d=32, F=16, E=8, k=3)
    x = rng.normal(size=(9, 32))
    out, ids, g, _ = oracle.moe_layer(L, x, n_threads=4)
    for t in range(9):
        o1, i1, g1, _ = oracle.moe_layer(L, x[t:t + 1])
        assert np.array_equal(o1[0], out[t]) and np.array_equal(i1[0], ids[t])


def test_decode_stack_chains_with_bf16_rounding():
    Ls = [tiny_layer(d=32, F=16, E=8, k=2, pre=True, seed=s)[1] for s in range(3)]
    x0 = oracle.round_bf16(rng.normal(size=32))
    li, out, ids, g, lg = oracle.decode_stack(Ls, x0, 2)
    cur = x0
    for t in range(2):
        for l in range(3):
            assert np.array_equal(li[t, l], cur)
            o, i, gg, _ = oracle.moe_layer(Ls[l], cur[None])
            assert np.array_equal(i[0], ids[t, l])
            cur = oracle.round_bf16(o[0])
        assert np.array_equal(out[t], cur)


# ---- rounding ---------------------------------------------------------------------------------------

def test_bf16_rounding_matches_library_on_fp32_values_and_avoids_double_rounding():
    v = rng.normal(size=5000).astype(np.float32)
    v = np.concatenate([v, v * 1e-30, v * 1e30, np.float32([0.0, -0.0, 3.0e38, 1e-40])])
    ours = oracle.round_bf16_bits(v.astype(np.float64))
    lib = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, lib)
    # halfway cases go to even
    assert oracle.round_bf16(np.array([1 + 2.0 ** -8]))[0] == 1.0
    assert oracle.round_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6
    # just above halfway: one rounding goes up (a detour through fp32 would tie and go down)
    assert oracle.round_bf16(np.array([1 + 2.0 ** -8 + 2.0 ** -30]))[0] == 1 + 2.0 ** -7


# ---- int8 spec mode ---------------------------------------------------------------------------------

def _exp_ulp_error(e, z):
    """Largest error of fp32 results e against the exponential of the fp32 arguments z, in units
    of the fp32 spacing at the exact value."""
    ref = np.exp(np.asarray(z, np.float64))
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    return float(np.max(np.abs(np.asarray(e, np.float64) - ref) / ulp))


def _degree6_expf(z):
    """A planted mistake, for the pin below to reject: the spec exp's steps with the r^7 term of
    the Taylor polynomial dropped (numpy fp32 operations, one rounding each)."""
    f = np.float32
    z = np.asarray(z, f)
    n = np.rint(z * f(1.4426950408889634))
    r = (z - n * f(0.693145751953125)) - n * f(0.6931471805599453 - 0.693145751953125)
    p = f(1.0 / 720.0)
    for c in (1.0 / 120.0, 1.0 / 24.0, 1.0 / 6.0, 0.5, 1.0, 1.0):
        p = p * r + f(c)
    return np.ldexp(p, n.astype(np.int32)).astype(f)


def test_spec_exp_accuracy_and_special_values():
    # a degree-7 Taylor polynomial after Cody-Waite reduction to |r| <= ln2/2 is within about one
    # ulp of e^z; 1.5 ulp is the pin.  Dropping the r^7 term (the planted variant) gives ~2.9 ulp
    # on this grid, so a lost Taylor term fails here.
    z = np.linspace(-80, 80, 200001).astype(np.float32)
    e = oracle.spec_expf(z).astype(np.float64)
    assert _exp_ulp_error(e, z) <= 1.5
    assert _exp_ulp_error(_degree6_expf(z), z) > 1.5
    assert oracle.spec_expf([0.0])[0] == 1.0
    assert np.all(np.diff(e) >= 0)
    # the reading's cutoffs: arguments above 80 give +inf, below -80 give 0 (no subnormal result);
    # 80 and -80 themselves are in range
    up = np.nextafter(np.float32(80), np.float32(np.inf))
    dn = np.nextafter(np.float32(-80), np.float32(-np.inf))
    big, small = oracle.spec_expf([80.0, -80.0])
    assert np.isfinite(big) and math.isclose(float(big), math.exp(80.0), rel_tol=2e-7)
    assert small > 0 and math.isclose(float(small), math.exp(-80.0), rel_tol=2e-7)
    assert oracle.spec_expf([up])[0] == np.inf and oracle.spec_expf([dn])[0] == 0.0
    assert oracle.spec_expf([81.0])[0] == np.inf and oracle.spec_expf([-81.0])[0] == 0.0
    for n in range(-100, 101, 7):
        zf = np.float32(n * math.log(2))              # the argument itself is rounded to fp32
        assert math.isclose(float(oracle.spec_expf([zf])[0]), math.exp(float(zf)), rel_tol=3e-7)
        assert math.isclose(float(oracle.spec_expf([zf])[0]), 2.0 ** n, rel_tol=abs(n) * 2e-7 + 3e-7)


def test_quant_absmax_closed_forms():
    xi = rng.integers(-126, 127, 300).astype(np.float32)
    xi[17] = -127.0
    q, s = oracle.quant_absmax(xi)
    assert s == 1.0 and np.array_equal(q.astype(np.float32), xi)
    q, s = oracle.quant_absmax(np.zeros(10, np.float32))
    assert s == 0.0 and np.all(q == 0)
    v = rng.normal(size=2048).astype(np.float32)
    q, s = oracle.quant_absmax(v)
    amax = np.abs(v).max()
    assert np.abs(q).max() == 127 and s == np.float32(amax / np.float32(127))
    assert np.max(np.abs(q - v.astype(np.float64) * 127 / amax)) <= 0.5 + 1e-5


def test_int8_accumulators_are_exact_integer_dots():
    w, L = tiny_layer(d=64, F=32, E=4, k=2)
    x = rng.integers(-127, 128, 64).astype(np.float32)
    x[3] = 127.0
    ids = np.array([3, 1], np.int32)
    g = np.array([0.75, 0.25], np.float32)
    out, taps = oracle.ffn_token_i8(L, x, ids, g)
    assert taps["sx"][0] == 1.0 and np.array_equal(taps["qx"].astype(np.float32), x)
    for j, e in enumerate(ids):
        assert np.array_equal(taps["acc_gate"][j], w["t_gate"][e].astype(np.int64) @ x.astype(np.int64))
        assert np.array_equal(taps["acc_up"][j], w["t_up"][e].astype(np.int64) @ x.astype(np.int64))
        assert np.array_equal(taps["acc_down"][j],
                              w["t_down"][e].astype(np.int64) @ taps["qh"][j].astype(np.int64))


def test_int8_spec_close_to_truth():
    w, L = tiny_layer(d=256, F=128, E=8, k=2, seed=9)
    x = rng.normal(size=(6, 256)).astype(np.float32)
    out_t, ids, g, _ = oracle.moe_layer(L, x)
    out_q = oracle.ffn_batch_i8(L, x, ids, g.astype(np.float32), n_threads=2)
    for t in range(6):
        ffn_t = out_t[t] - x[t]
        ffn_q = out_q[t].astype(np.float64) - x[t]
        assert np.max(np.abs(ffn_q - ffn_t)) / np.max(np.abs(ffn_t)) < 5e-2


def test_int8_all_zero_codes_and_zero_input():
    w, L = tiny_layer(d=32, F=16, E=4, k=2)
    x = rng.normal(size=32).astype(np.float32)
    z = dict(w, t_gate=np.zeros_like(w["t_gate"]), t_up=np.zeros_like(w["t_up"]),
             t_down=np.zeros_like(w["t_down"]))
    out, _ = oracle.ffn_token_i8(oracle.Layer(**z, top_k=2), x, [0, 1], [0.5, 0.5])
    assert np.array_equal(out, x)
    out, taps = oracle.ffn_token_i8(L, np.zeros(32, np.float32), [0, 1], [0.5, 0.5])
    assert np.all(out == 0) and taps["sx"][0] == 0


# ---- the pages' printed numbers -----------------------------------------------------------------

def test_bandwidth_worked_example_from_the_pages():
    ex = json.load(open(os.path.join(GOLDEN, "bandwidth_example.json")))
    rate = accounting.ceiling_rate(ex["bytes_per_token"], ex["bandwidth_bytes_per_s"])
    assert round(1e3 / rate, 2) == ex["ms_per_token"]
    assert round(rate) == ex["ceiling_tok_s"]
    frac = accounting.fraction_of_peak(ex["measured_tok_s"], ex["bytes_per_token"],
                                       ex["bandwidth_bytes_per_s"])
    assert round(frac, 2) == ex["fraction_of_peak"]


def test_ternary_size_example_from_the_pages():
    ex = json.load(open(os.path.join(GOLDEN, "ternary_size_example.json")))
    assert round(math.log2(3), 3) == ex["bits_per_state_ideal"]
    assert round(ex["params"] * math.log2(3) / 8 / 1e9, 2) * 1e9 == ex["bytes_ideal"]
    # the 2-bit packing used here: four weights per byte
    w = rand_trits(1, 4000)
    assert oracle.pack(w)[0].size * ex["weights_per_byte"] == 4000
    assert ex["params"] * 2 == ex["bytes_bf16"]


def test_workload_byte_accounting():
    # one full-size layer at batch 1 and the 24-layer stack (expert codes + scales + router + I/O)
    assert accounting.layer_bytes(synth.LAYER_B1) == 7_446_528
    assert accounting.stack_bytes_per_token(synth.STACK24_B1) == 178_716_672
    assert 24 * 8 * 786_432 == 150_994_944      # expert codes per token in the stack
    assert accounting.layer_bytes(synth.SMALL_LAYER_B1) == 2 * 26_624 + 16_384 + 2 * 1024


# ---- float -> ternary quantisation (per-row absmean) --------------------------------------------

def test_quantize_equal_magnitudes_give_signs_and_that_magnitude():
    # every |w| = 2^-3: the mean is exactly 2^-3, w / g = +-1
    signs = np.where(rng.random((5, 2048)) < 0.5, -1.0, 1.0).astype(np.float32)
    t, s = oracle.quantize_absmean(signs * 0.125)
    assert np.array_equal(t, signs.astype(np.int8))
    assert np.all(s == np.float32(0.125))


@pytest.mark.parametrize("cols", [8, 512, 2048, 2056])
def test_quantize_scaled_trits_round_trip(cols):
    # w = a * T with a = 2^-5: the absolute sum a * nnz is exact in any order, g = a nnz / cols
    # (a power-of-two cols divides exactly; 2056 = 8 * 257 checked against the exact quotient),
    # and |w| / g = cols / nnz >= 1 for every nonzero, so the codes reproduce T
    T = rand_trits(6, cols)
    T[0] = 0
    T[0, 3] = -1          # a single nonzero: |w| / g = cols
    T[1] = 1              # all +1: g = a
    t, s = oracle.quantize_absmean(T.astype(np.float32) * np.float32(2.0 ** -5))
    nnz = np.count_nonzero(T, axis=1)
    assert np.array_equal(t, T)
    assert np.array_equal(s, (np.float32(2.0 ** -5) * nnz.astype(np.float32)) / np.float32(cols))
    assert s[1] == np.float32(2.0 ** -5)


def test_quantize_zero_row():
    w = np.zeros((2, 64), np.float32)
    w[1, 5] = 3.0
    t, s = oracle.quantize_absmean(w)
    assert np.all(t[0] == 0) and s[0] == 0.0
    assert t[1, 5] == 1 and np.count_nonzero(t[1]) == 1 and s[1] == np.float32(3.0 / 64)


def test_quantize_threshold_and_ties_to_even():
    # cols 8: seven entries 15 and one v give g = (105 + |v|) / 8.  v = +-7: g = 14 and v / g =
    # +-0.5 exactly, which rounds to 0 (ties to even); 15 / 14 rounds to 1.  v = 1.875: g =
    # 3.734375, v / g = 0.502 -> 1 (against seven 4s); v = 1.75 -> 0.4706 -> 0.  v = 21 against
    # seven 1s: g = 3.5, 21 / 3.5 = 6 -> clamped to 1.
    w = np.array([[15] * 7 + [7], [15] * 7 + [-7], [4] * 7 + [1.875], [4] * 7 + [1.75],
                  [1] * 7 + [21], [-1] * 7 + [-21]], np.float32)
    t, s = oracle.quantize_absmean(w)
    assert t[:, 7].tolist() == [0, 0, 1, 0, 1, -1]
    assert t[0, :7].tolist() == [1] * 7 and t[5, :7].tolist() == [0] * 7
    assert s.tolist() == [14.0, 14.0, 3.734375, 3.71875, 3.5, 3.5]


def test_quantize_scale_is_the_correctly_rounded_mean_magnitude():
    # the exact mean of |w| (rational arithmetic) rounded once to fp32: the scale is within half an
    # fp32 ulp of it (a slack of 2^-28 ulp covers the double-precision sum)
    from fractions import Fraction
    w = (rng.normal(0, 0.02, (16, 2048))).astype(np.float32)
    w[3] *= 1e-20
    _, s = oracle.quantize_absmean(w)
    for r in range(w.shape[0]):
        exact = sum((Fraction(float(v)) for v in np.abs(w[r])), Fraction(0)) / w.shape[1]
        err = abs(Fraction(float(s[r])) - exact)
        half_ulp = Fraction(float(np.spacing(np.float32(float(exact))))) / 2
        assert err <= half_ulp * (1 + Fraction(1, 2 ** 28)), r


def test_quantize_is_independent_of_column_order():
    # a mean has no order: permuting a row's weights permutes its codes and keeps its scale
    w = (rng.normal(0, 0.02, (8, 2048))).astype(np.float32)
    perm = rng.permutation(2048)
    t, s = oracle.quantize_absmean(w)
    tp, sp = oracle.quantize_absmean(w[:, perm])
    assert np.array_equal(s, sp) and np.array_equal(tp, t[:, perm])


def test_quantize_rows_of_any_length():
    # rows that are not a multiple of 8: three weights 3, -1, 0.5 -> g = 1.5; 3/1.5 = 2 -> 1,
    # -1/1.5 -> -0.67 -> -1, 0.5/1.5 = 0.33 -> 0; an empty row set is a no-op
    t, s = oracle.quantize_absmean(np.array([[3.0, -1.0, 0.5]], np.float32))
    assert t.tolist() == [[1, -1, 0]] and s.tolist() == [1.5]
    t, s = oracle.quantize_absmean(np.zeros((0, 5), np.float32))
    assert t.shape == (0, 5) and s.shape == (0,)


def test_quantize_neighbours_of_the_half_scale():
    # seven 15s and v = 7 (1 ulp up/down): the mean (105 + v) / 8 rounds to 14 either way, g = 14,
    # and v / g rounds above 1/2 (code 1) for the next float above 7, to 1/2 exactly (code 0, ties
    # to even) for 7, below 1/2 (code 0) for the float below 7
    up, dn = np.nextafter(np.float32(7), np.float32(8)), np.nextafter(np.float32(7), np.float32(6))
    w = np.array([[15] * 7 + [up], [15] * 7 + [7], [15] * 7 + [dn], [15] * 7 + [-up]], np.float32)
    t, s = oracle.quantize_absmean(w)
    assert s.tolist() == [14.0] * 4
    assert t[:, 7].tolist() == [1, 0, 0, -1]


# ---- base-3 packing (five weights per byte) and the int8 GEMV spec ------------------------------

def test_pack3_worked_bytes():
    # byte = sum_i (w_i + 1) 3^i, weight 5j the least significant trit; padding counts as weight 0
    p, bad = oracle.pack3(np.array([[1, 0, -1, 1, 1, 0, -1]], np.int8), 16)
    assert bad == 0
    assert p[0, 0] == 2 * 1 + 1 * 3 + 0 * 9 + 2 * 27 + 2 * 81        # 221
    assert p[0, 1] == 1 * 1 + 0 * 3 + 1 * 9 + 1 * 27 + 1 * 81        # 118: w5 = 0, w6 = -1, 3 pads
    assert not p[0, 2:].any()                                          # bytes past ceil(7/5)
    assert oracle.pack3(np.ones((1, 5), np.int8))[0][0, 0] == 242
    assert oracle.pack3(-np.ones((1, 5), np.int8))[0][0, 0] == 0
    assert oracle.pack3(np.zeros((1, 5), np.int8))[0][0, 0] == 121


def test_pack3_is_a_bijection_on_all_243_groups():
    import itertools
    groups = np.array(list(itertools.product([-1, 0, 1], repeat=5)), np.int8)   # 243 x 5
    p, bad = oracle.pack3(groups)
    assert bad == 0 and p.shape == (243, 1)
    assert sorted(p[:, 0].tolist()) == list(range(243))
    # digit-by-digit division by 3 (textbook base conversion) recovers each weight
    for g, b in zip(groups, p[:, 0]):
        v = int(b)
        for i in range(5):
            assert v % 3 - 1 == g[i]
            v //= 3
    w, bad = oracle.unpack3(p, 5)
    assert bad == 0 and np.array_equal(w, groups)


@pytest.mark.parametrize("cols", [1, 4, 5, 6, 2048, 2051])
def test_pack3_round_trip_and_size(cols):
    w = rand_trits(3, cols)
    rb = ((cols + 4) // 5 + 15) // 16 * 16
    p, bad = oracle.pack3(w, rb)
    assert bad == 0 and p.shape == (3, rb)
    assert not p[:, (cols + 4) // 5:].any()
    back, bad = oracle.unpack3(p, cols)
    assert bad == 0 and np.array_equal(back, w)


def test_pack3_counts_and_zeroes_invalid_values_and_bytes():
    w = np.array([[2, 1, -5, 0, 1]], np.int8)
    p, bad = oracle.pack3(w)
    assert bad == 2
    assert np.array_equal(oracle.unpack3(p, 5)[0], np.array([[0, 1, 0, 0, 1]], np.int8))
    back, bad = oracle.unpack3(np.array([[243, 242, 255]], np.uint8), 15)
    assert bad == 2 and not back[0, :5].any() and (back[0, 5:10] == 1).all() and not back[0, 10:].any()


def test_pack3_size_against_the_information_bound():
    # five trits per byte: 1.6 bits per weight against log2 3 = 1.585 (within 1%); a 2048-weight
    # row takes 410 bytes (416 at a 16-byte row stride) against 512 at four weights per byte
    ex = json.load(open(os.path.join(GOLDEN, "ternary_size_example.json")))
    assert 3 ** 5 <= 256 < 3 ** 6
    assert 8 / 5 / ex["bits_per_state_ideal"] < 1.01
    assert oracle.pack3(rand_trits(1, 2048))[0].shape[1] == 410
    assert oracle.pack(rand_trits(1, 2048))[0].shape[1] == 512


def test_gemv_i8_integer_sums_are_brute_force_dots():
    # sx = scale = 1: y is the exact integer dot (|sum| < 2^24), checked against Python integers
    w = rand_trits(7, 53)
    q = rng.integers(-127, 128, 53).astype(np.int8)
    y = oracle.gemv_i8(w, np.ones(7, np.float32), q, 1.0)
    for r in range(7):
        assert y[r] == sum(int(a) * int(b) for a, b in zip(w[r], q))


def test_gemv_i8_one_hot_rows_sign_symmetry_and_power_of_two_scales():
    cols = 40
    q = rng.integers(-127, 128, cols).astype(np.int8)
    w = np.zeros((cols, cols), np.int8)
    w[np.arange(cols), np.arange(cols)] = 1                           # row r picks input r
    s = np.full(cols, 0.25, np.float32)
    y = oracle.gemv_i8(w, s, q, 2.0)
    assert np.array_equal(y, q.astype(np.float32) * 0.5)             # exact: powers of two
    w2 = rand_trits(9, cols)
    s2 = rng.uniform(0.01, 1.0, 9).astype(np.float32)
    assert np.array_equal(oracle.gemv_i8(-w2, s2, q, 0.37), -oracle.gemv_i8(w2, s2, q, 0.37))


def test_gemv_i8_matches_the_int8_ffn_gate_accumulators():
    # the gate rows of the int8 FFN spec: its tapped integer sums times sx times the row scales,
    # in that order, are what gemv_i8 gives on the same rows
    w, L = tiny_layer(d=64, F=32, E=4, k=2)
    x = rng.normal(0, 1, 64).astype(np.float32)
    ids = np.array([2, 0], np.int32)
    out, taps = oracle.ffn_token_i8(L, x, ids, np.array([0.5, 0.5], np.float32))
    for j, e in enumerate(ids):
        y = oracle.gemv_i8(w["t_gate"][e], w["s_gate"][e], taps["qx"], taps["sx"][0])
        ref = (taps["acc_gate"][j].astype(np.float32) * np.float32(taps["sx"][0])) * \
            w["s_gate"][e].astype(np.float32)
        assert np.array_equal(y, ref)


# ---- decode attention over a KV cache (grouped-query, global or ring-buffered window) ------------

def test_attention_single_position_returns_its_value():
    q = rng.normal(size=(8, 16))
    k = rng.normal(size=(1, 2, 16))
    v = rng.normal(size=(1, 2, 16))
    o = oracle.attention_decode(q, k, v)
    for h in range(8):
        assert np.array_equal(o[h], v[0, h // 4])      # 4 query heads per KV head


def test_attention_equal_scores_average_the_values():
    # zero query (or identical keys): uniform weights, the output is the mean of the values
    v = rng.normal(size=(10, 2, 8))
    o = oracle.attention_decode(np.zeros((4, 8)), rng.normal(size=(10, 2, 8)), v)
    assert np.allclose(o[0], v[:, 0].mean(axis=0), rtol=0, atol=1e-14)
    assert np.allclose(o[3], v[:, 1].mean(axis=0), rtol=0, atol=1e-14)
    k = np.repeat(rng.normal(size=(1, 2, 8)), 10, axis=0)
    o2 = oracle.attention_decode(rng.normal(size=(4, 8)), k, v)
    assert np.allclose(o2[1], v[:, 0].mean(axis=0), rtol=0, atol=1e-14)


def test_attention_dominant_key_selects_its_value():
    dh = 8
    k = np.zeros((6, 1, dh))
    k[4, 0, 0] = 100.0
    q = np.zeros((1, dh))
    q[0, 0] = 100.0                      # score 10000 / sqrt(8) against 0 for the others
    v = rng.normal(size=(6, 1, dh))
    assert np.allclose(oracle.attention_decode(q, k, v)[0], v[4, 0], rtol=0, atol=1e-300)


def test_attention_matches_library_softmax_and_sdpa():
    H, Hkv, dh, n = 16, 4, 128, 37
    q = rng.normal(size=(H, dh))
    k = rng.normal(size=(n, Hkv, dh))
    v = rng.normal(size=(n, Hkv, dh))
    o = oracle.attention_decode(q, k, v)
    qt = torch.from_numpy(q)[:, None, :]                                     # [H][1][dh]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(H // Hkv, 0)  # [H][n][dh]
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(H // Hkv, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[:, 0, :].numpy()
    assert np.allclose(o, ref, rtol=0, atol=1e-12)
    w = torch.softmax(torch.einsum("hd,hnd->hn", qt[:, 0], kt) / math.sqrt(dh), dim=1)
    assert np.allclose(o, torch.einsum("hn,hnd->hd", w, vt).numpy(), rtol=0, atol=1e-12)


def test_attention_ring_order_does_not_matter():
    # a windowed layer's ring holds its last positions in rotated slot order
    q = rng.normal(size=(4, 32))
    k = rng.normal(size=(20, 2, 32))
    v = rng.normal(size=(20, 2, 32))
    rot = np.roll(np.arange(20), 7)
    assert np.allclose(oracle.attention_decode(q, k, v), oracle.attention_decode(q, k[rot], v[rot]),
                       rtol=0, atol=1e-13)


# ---- approximate output head: 4-bit centroid scores, top clusters, exact logits -----------------

def pack_nibbles(vals):
    """values -8..7 [..., d] -> offset nibbles, element 2k low and 2k+1 high in byte k"""
    u = (np.asarray(vals, np.int64) + 8).astype(np.uint8)
    return (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)


def flash_inputs(d=64, ncl=20, cs=4, seed=3):
    r = np.random.default_rng(seed)
    vals = r.integers(-8, 8, (ncl, d))
    return dict(h=r.normal(0, 1, d).astype(np.float32), vals=vals, cent=pack_nibbles(vals),
                cscale=r.uniform(0.01, 0.1, ncl).astype(np.float32),
                wc=r.normal(0, 0.02, (ncl, cs, d)).astype(np.float32),
                members=r.permutation(ncl * cs).astype(np.int32).reshape(ncl, cs))


def test_flash_head_scores_are_exact_integer_dots_of_the_centroids():
    f = flash_inputs()
    sel, ids, lg, scores = oracle.flash_head(f["h"], f["cent"], f["cscale"], f["wc"], f["members"], 5)
    q, sh = oracle.quant_absmax(f["h"])
    acc = f["vals"].astype(np.int64) @ q.astype(np.int64)           # brute-force integer dots
    assert np.array_equal(scores, (acc.astype(np.float32) * np.float32(sh)) * f["cscale"])
    # a one-hot centroid row scores its single value times that input's code
    v = np.zeros((1, 64), np.int64)
    v[0, 9] = -7
    s1 = oracle.flash_head(f["h"], pack_nibbles(v), np.ones(1, np.float32), f["wc"][:1],
                           f["members"][:1], 1)[3]
    assert s1[0] == np.float32(np.float32(-7 * int(q[9])) * np.float32(sh))


def test_flash_head_selection_matches_library_sort_with_ties_to_lower_ids():
    f = flash_inputs(ncl=30)
    q, _ = oracle.quant_absmax(f["h"])
    best = np.where(q > 0, 7, -8)[None, :]        # the largest possible score for this input
    f["cent"][3] = f["cent"][7] = pack_nibbles(best)[0]
    f["cscale"][3] = f["cscale"][7] = 0.5
    sel, ids, lg, scores = oracle.flash_head(f["h"], f["cent"], f["cscale"], f["wc"], f["members"], 12)
    ref = np.lexsort((np.arange(30), -scores.astype(np.float64)))[:12]
    assert np.array_equal(sel, ref)
    assert scores[3] == scores[7] and sel[0] == 3 and sel[1] == 7


def test_flash_head_logits_match_library_matmul_and_member_ids():
    f = flash_inputs()
    sel, ids, lg, scores = oracle.flash_head(f["h"], f["cent"], f["cscale"], f["wc"], f["members"], 6)
    ref = np.einsum("jmd,d->jm", f["wc"][sel].astype(np.float64), f["h"].astype(np.float64))
    assert np.allclose(lg, ref, rtol=0, atol=1e-13)
    assert np.array_equal(ids, f["members"][sel])


def test_flash_head_with_every_cluster_is_the_exact_head():
    # selecting all clusters covers the whole vocabulary: the best logit is the exact head's argmax
    f = flash_inputs(ncl=16, cs=8)
    sel, ids, lg, scores = oracle.flash_head(f["h"], f["cent"], f["cscale"], f["wc"], f["members"], 16)
    assert sorted(ids.reshape(-1).tolist()) == list(range(128))
    W = np.empty((128, 64))
    W[f["members"].reshape(-1)] = f["wc"].reshape(128, 64)
    full = W @ f["h"].astype(np.float64)
    assert ids.reshape(-1)[np.argmax(lg.reshape(-1))] == np.argmax(full)
    assert np.isclose(lg.max(), full.max(), rtol=0, atol=1e-13)
