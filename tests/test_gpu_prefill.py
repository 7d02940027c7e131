"""Parity of the grouped MFMA path (many tokens per expert, prefill-shaped) with the CPU oracle's
int8 specification and with the per-pair v_dot4 path, bit for bit.  The int8 path is exact, so the
three must agree in every bit of the fp32 output.  Routing is an input (computed by moe_route_topk
on the GPU and handed to both sides).  The two-plane (bf16) tiles are checked against the small-tile
path bit for bit and against the oracle's truth mode; fp32 inputs are checked on the v_dot4 path."""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
import ternary_weight_moe_amd as tw
from parity_util import LayerPair, make_pair, require_gpu, step

pytestmark = pytest.mark.gpu

NTH = min(16, os.cpu_count() or 1)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.fixture(scope="module")
def full():
    step("build layer_b1 layer pair (full size) for the prefill tests")
    return make_pair(synth.LAYER_B1)


def run_int8(layer, x, ids, gates):
    out = tw.ternary_moe_ffn_batched(layer, x, act="int8", out_dtype=torch.float32,
                                     expert_ids=ids, gate_w=gates)
    torch.cuda.synchronize()
    return out


def dot_path_in_chunks(layer, x, ids, gates, chunk=64):
    """The same tokens through calls small enough to take the per-pair v_dot4 path."""
    outs = [run_int8(layer, x[i:i + chunk].contiguous(), ids[i:i + chunk].contiguous(),
                     gates[i:i + chunk].contiguous()) for i in range(0, x.shape[0], chunk)]
    return torch.cat(outs)


def bits(t):
    return t.cpu().numpy().view(np.uint32)


def test_prefill_int8_matches_oracle_and_dot_path(full):
    T = 256   # T*k = 8*E: the grouped MFMA path
    x = synth.activations(synth.PREFILL_4096, T, seed=71).cuda()
    _, ids, gates = tw.moe_route_topk(x, full.gpu.w_router, 8)
    step("prefill int8 T=%d (MFMA path)" % T)
    out = run_int8(full.gpu, x, ids, gates)
    step("same tokens through the dot4 path")
    ref_dot = dot_path_in_chunks(full.gpu, x, ids, gates)
    assert np.array_equal(bits(out), bits(ref_dot))
    step("oracle int8 spec, %d tokens, %d threads" % (T, NTH))
    ref = oracle.ffn_batch_i8(full.ora, x.cpu(), ids.cpu().numpy(), gates.cpu().numpy(),
                              n_threads=NTH)
    assert np.array_equal(bits(out), ref.view(np.uint32))


def test_prefill_int8_full_size(full):
    # 4096 tokens, top-8 of 256 experts (~128 per expert): every output against the dot4 path,
    # a sample of tokens against the oracle
    T = 4096
    x = synth.activations(synth.PREFILL_4096, T).cuda()
    _, ids, gates = tw.moe_route_topk(x, full.gpu.w_router, 8)
    step("prefill int8 T=4096 (MFMA path)")
    out = run_int8(full.gpu, x, ids, gates)
    step("4096 tokens through the dot4 path in 64-token calls")
    ref_dot = dot_path_in_chunks(full.gpu, x, ids, gates)
    assert np.array_equal(bits(out), bits(ref_dot))
    sample = np.unique(np.concatenate([np.arange(0, T, 97), [1, 63, 64, T - 2, T - 1]]))
    step("oracle int8 spec on %d sampled tokens" % len(sample))
    ref = oracle.ffn_batch_i8(full.ora, x.cpu()[sample], ids.cpu().numpy()[sample],
                              gates.cpu().numpy()[sample], n_threads=NTH)
    assert np.array_equal(bits(out)[sample], ref.view(np.uint32))


def test_prefill_int8_one_hot_experts_ragged_tiles(full):
    # every token sends its 8 slots to the same 8 experts: 1000 tokens per expert, 15 full tiles
    # of 64 and a 40-token tail each
    T = 1000
    x = synth.activations(synth.PREFILL_4096, T, seed=73).cuda()
    ids = torch.tensor([3, 250, 17, 0, 128, 255, 64, 9], dtype=torch.int32).repeat(T, 1).cuda()
    g = torch.rand((T, 8), generator=torch.Generator().manual_seed(5)) + 0.05
    gates = (g / g.sum(1, keepdim=True)).float().contiguous().cuda()
    step("prefill int8 adversarial routing T=1000")
    out = run_int8(full.gpu, x, ids, gates)
    ref_dot = dot_path_in_chunks(full.gpu, x, ids, gates)
    assert np.array_equal(bits(out), bits(ref_dot))
    sample = np.array([0, 1, 959, 960, 999])
    ref = oracle.ffn_batch_i8(full.ora, x.cpu()[sample], ids.cpu().numpy()[sample],
                              gates.cpu().numpy()[sample], n_threads=NTH)
    assert np.array_equal(bits(out)[sample], ref.view(np.uint32))


@pytest.mark.parametrize("T", [1024, 3072])
def test_prefill_int8_bf16_output_is_the_fp32_result_rounded(full, T):
    # The 16-bit down sums of the grouped kernels (64-token tiles at 1024 tokens, one work item per
    # expert at 3072) with bf16 output: the combine rounds its fp32 result once, so every output is
    # the fp32 output of the same call rounded to bf16 (the fp32 output is pinned to the oracle and
    # the v_dot4 path by the tests above)
    x = synth.activations(synth.PREFILL_4096, T, seed=79).cuda()
    _, ids, gates = tw.moe_route_topk(x, full.gpu.w_router, 8)
    step("prefill int8 T=%d, fp32 and bf16 outputs" % T)
    out32 = run_int8(full.gpu, x, ids, gates)
    out16 = tw.ternary_moe_ffn_batched(full.gpu, x, act="int8", out_dtype=torch.bfloat16,
                                       expert_ids=ids, gate_w=gates)
    torch.cuda.synchronize()
    ref16 = oracle.round_bf16_bits(out32.cpu().numpy().astype(np.float64))
    assert np.array_equal(out16.cpu().view(torch.int16).numpy().view(np.uint16), ref16)
    sample = np.array([0, T // 2, T - 1])
    ref = oracle.ffn_batch_i8(full.ora, x.cpu()[sample], ids.cpu().numpy()[sample],
                              gates.cpu().numpy()[sample], n_threads=NTH)
    assert np.array_equal(bits(out32)[sample], ref.view(np.uint32))


def skewed_ids(T, E, k, seed):
    """Top-k ids with a heavy skew: slot 0 always expert 7, the other slots drawn without
    replacement from 200 other experts (shuffled) with weights 1 / (rank + 1), so that per-expert
    counts range from thousands to a handful, and E - 201 experts get none."""
    rng = np.random.default_rng(seed)
    order = rng.permutation([e for e in range(E) if e != 7])[:200]
    p = 1.0 / (np.arange(len(order)) + 1.0)
    p /= p.sum()
    ids = np.empty((T, k), np.int32)
    ids[:, 0] = 7
    for i in range(T):
        ids[i, 1:] = rng.choice(order, size=k - 1, replace=False, p=p)
    return ids


def test_prefill_int8_expert_items_skewed_counts(full):
    # 4096 tokens, one work item per (expert, up to 176 tokens): expert 7 takes every token (24
    # items, the last of 48 tokens), the rest range from hundreds of tokens to a handful or none,
    # so items of every size class run side by side
    T = 4096
    x = synth.activations(synth.PREFILL_4096, T, seed=77).cuda()
    ids_np = skewed_ids(T, 256, 8, seed=9)
    counts = np.bincount(ids_np.ravel(), minlength=256)
    rem = counts[counts > 0] % 176
    # last items of every size class (16-token row blocks: up to 4, 5-8, 9, 10, 11)
    for lo, hi in [(0, 16), (16, 64), (64, 128), (128, 144), (144, 160), (160, 175)]:
        assert ((rem > lo) & (rem <= hi)).any(), (lo, hi)
    assert counts.max() == T and (counts == 0).sum() == 256 - 201
    ids = torch.from_numpy(ids_np).cuda()
    g = torch.rand((T, 8), generator=torch.Generator().manual_seed(6)) + 0.05
    gates = (g / g.sum(1, keepdim=True)).float().contiguous().cuda()
    step("prefill int8 skewed routing T=4096 (one item per expert)")
    out = run_int8(full.gpu, x, ids, gates)
    step("4096 tokens through the dot4 path in 64-token calls")
    ref_dot = dot_path_in_chunks(full.gpu, x, ids, gates)
    assert np.array_equal(bits(out), bits(ref_dot))
    sample = np.array([0, 1, 175, 176, 2047, T - 1])
    step("oracle int8 spec on %d sampled tokens" % len(sample))
    ref = oracle.ffn_batch_i8(full.ora, x.cpu()[sample], ids_np[sample], gates.cpu().numpy()[sample],
                              n_threads=NTH)
    assert np.array_equal(bits(out)[sample], ref.view(np.uint32))


@pytest.mark.parametrize("T", [256, 1024, 2048])
def test_prefill_int8_second_shape(T):
    # d=1024, 64 experts, F=256, top-4: the second instantiation of the MFMA path; 256 tokens take
    # the small self-grouped tiles, 1024 tokens (64 pairs per expert) the 64-token tiles, whose
    # ragged last tiles of at most 32 tokens take the half-size body, and 2048 tokens (128 pairs per
    # expert) one work item per (expert, up to 176 tokens)
    wl = synth.MID_STACK_B1
    pair = make_pair(wl, pre=False)
    x = synth.activations(wl, T, seed=75).cuda()
    _, ids, gates = tw.moe_route_topk(x, pair.gpu.w_router, wl.top_k)
    step("prefill int8 mid shape T=%d" % T)
    out = run_int8(pair.gpu, x, ids, gates)
    ref = oracle.ffn_batch_i8(pair.ora, x.cpu(), ids.cpu().numpy(), gates.cpu().numpy(),
                              n_threads=NTH)
    assert np.array_equal(bits(out), ref.view(np.uint32))
    ref_dot = dot_path_in_chunks(pair.gpu, x, ids, gates)
    assert np.array_equal(bits(out), bits(ref_dot))


def run_float(layer, x, ids, gates):
    out = tw.ternary_moe_ffn_batched(layer, x, act="float", expert_ids=ids, gate_w=gates)
    torch.cuda.synchronize()
    return out


def test_batched_bf16_large_tiles_match_small_tiles(full):
    # 1024 bf16 tokens (32 pairs per expert on average): 32-token tiles of two digit planes; the same
    # tokens in 64-token calls take 8-token tiles.  The ternary sums are exact integer sums of the same
    # digits, so both give the same bits; a sample is also checked against the oracle.
    T = 1024
    x = synth.activations(synth.BATCHED_B64, T, seed=91).cuda()
    _, ids, gates = tw.moe_route_topk(x, full.gpu.w_router, 8)
    step("batched bf16 T=%d (32-token tiles)" % T)
    out = run_float(full.gpu, x, ids, gates)
    step("same tokens in 64-token calls (8-token tiles)")
    ref = torch.cat([run_float(full.gpu, x[i:i + 64].contiguous(), ids[i:i + 64].contiguous(),
                               gates[i:i + 64].contiguous()) for i in range(0, T, 64)])
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    step("oracle truth mode on sampled tokens")
    xs = x.cpu()
    ids_np, g_np = ids.cpu().numpy(), gates.cpu().numpy()
    for t in (0, 1, 511, T - 1):
        o = oracle.ffn_token(full.ora, xs[t].double().numpy(), ids_np[t], g_np[t].astype(np.float64))
        got = out[t].float().cpu().numpy()
        assert np.max(np.abs(got - o)) <= 2e-2 * np.max(np.abs(o)), t


def test_batched_fp32_input_served_by_dot4_kernels(full):
    # fp32 activations need three digit planes, which the grouped MFMA kernel does not take: the
    # per-pair v_dot4 kernels serve the call
    T = 16
    x = synth.activations(synth.BATCHED_B64, T, seed=93).float()
    oids, og, _ = oracle.route(full.ora, x, n_threads=8)
    ids = torch.from_numpy(oids).cuda()
    gates = torch.from_numpy(og.astype(np.float32)).cuda()
    step("batched fp32 input T=%d" % T)
    out = run_float(full.gpu, x.cuda(), ids, gates)
    for t in range(T):
        o = oracle.ffn_token(full.ora, x[t].double().numpy(), oids[t], og[t])
        got = out[t].cpu().numpy()
        assert np.max(np.abs(got - o)) <= 1e-4 * np.max(np.abs(o)), t


@pytest.mark.parametrize("T", [40, 300])
def test_batched_int8_invalid_slots_contribute_nothing(full, T):
    # slots whose expert id is outside [0, E) contribute nothing; a token with no valid slot gets
    # out = x.  Expected: the oracle's int8 spec with those slots given gate 0 (an exact zero term)
    # and a valid id.  T = 40: small tiles built in every workgroup; T = 300: k_group's tiles
    x = synth.activations(synth.PREFILL_4096, T, seed=81).cuda()
    _, ids, gates = tw.moe_route_topk(x, full.gpu.w_router, 8)
    ids, gates = ids.clone(), gates.clone()
    r = np.random.default_rng(T)
    bad = torch.as_tensor(r.random(ids.shape) < 0.2, device=ids.device)
    bad[5] = True                                   # token 5: no valid slot
    bad[7] = False
    badval = torch.as_tensor(r.choice([-1, 256, 1000, -7], ids.shape), device=ids.device,
                             dtype=ids.dtype)
    ids = torch.where(bad, badval, ids)
    step("batched int8 with invalid slots, T=%d" % T)
    out = run_int8(full.gpu, x, ids, gates)
    ids_o = torch.where(bad, torch.zeros_like(ids), ids).cpu().numpy()
    gates_o = torch.where(bad, torch.zeros_like(gates), gates).cpu().numpy()
    ref = oracle.ffn_batch_i8(full.ora, x.cpu(), ids_o, gates_o, n_threads=NTH)
    assert np.array_equal(bits(out), ref.view(np.uint32))
    assert torch.equal(out[5], x[5].float())


@pytest.mark.parametrize("T,E,k", [(40, 8, 4), (150, 8, 4), (300, 8, 4), (300, 16, 8)])
def test_int8_down_sums_outside_int16(T, E, k):
    # With int8 activations in 64-token tiles the grouped kernel keeps each down sum as an int16 and
    # marks the ones outside [-32767, 32767], which then come from 32-bit rows.  Expert 0 here has all-+1 gate and
    # up rows with equal scales, and every input of the tokens is positive, so its h is the same
    # value in all F rows and quantises to 127 everywhere; its down row r has +1 in the first
    # r mod 513 positions and -1 after them, so the down sums are 127 (2 a - 512) for every a in
    # 0 .. 512: from -65024 to 65024, with 32766 the largest that fits and 33020 the smallest that
    # does not.  Expected: the oracle's int8 spec bit for bit.  T = 40: small self-grouped tiles
    # (fp32 y rows); T = 150: 64-token tiles from the grouping kernel (16-bit sums); T = 300 (at
    # least 96 pairs per expert): one work item per (expert, up to 176 tokens), also 16-bit sums,
    # top-4 (the combine's slot count given at run time) and top-8 (fixed when compiled).
    wl = synth.PREFILL_4096
    d, F = wl.d_model, wl.d_ff
    w = synth.layer_weights(wl, 0, n_experts=E)
    w["t_gate"][0] = 1
    w["t_up"][0] = 1
    w["s_gate"][0] = 0.03
    w["s_up"][0] = 0.02
    a = torch.arange(d).remainder(F + 1)
    w["t_down"][0] = torch.where(torch.arange(F)[None, :] < a[:, None], 1, -1).to(torch.int8)
    pair = LayerPair(w, k, False)
    x = (synth.activations(wl, T, seed=83).float().abs() + 0.25).to(torch.bfloat16)
    r = np.random.default_rng(T)
    ids_np = np.stack([np.concatenate([[0], r.permutation(np.arange(1, E))[:k - 1]]) for _ in range(T)])
    g = r.random((T, k)) + 0.05
    gates_np = (g / g.sum(1, keepdims=True)).astype(np.float32)
    sums = 127 * (2 * a.numpy() - F)
    assert (np.abs(sums) > 32767).sum() > 500 and (np.abs(sums) <= 32767).sum() > 500
    step("batched int8 with down sums outside int16, T=%d" % T)
    out = run_int8(pair.gpu, x.cuda(), torch.from_numpy(ids_np.astype(np.int32)).cuda(),
                   torch.from_numpy(gates_np).cuda())
    ref = oracle.ffn_batch_i8(pair.ora, x, ids_np.astype(np.int32), gates_np, n_threads=NTH)
    assert np.array_equal(bits(out), ref.view(np.uint32))
