"""Decode attention over a KV cache on the GPU through the C ABI, against the CPU oracle (fp64):
grouped-query heads, the pages' 640-token global context and 512-slot window, ragged slot counts
around the 16-slot splits, long contexts, sharp softmaxes and rotated ring slots, and a reused
workspace.

Tolerance: the kernel sums in fp32 (128-term score dots, 64-slot value sums per split, a merge over
splits), so each score carries a relative error of about 128 x 2^-24 of sum |q_i k_i| (about 6e-5
absolute for N(0,1) rows scaled by 1/sqrt(128)), which moves each softmax weight by the same
relative amount; the output error is then bounded by about 1e-4 of max |v|.  The test requires
max |gpu - oracle| <= 1e-4 * max |oracle| per call (normwise), and reports the margin."""
import numpy as np
import pytest
import torch

import oracle
import synth
import ternary_weight_moe_amd as tw
from parity_util import require_gpu, step

pytestmark = pytest.mark.gpu
TOL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def check(q, k, v, out):
    ref = oracle.attention_decode(q.float().cpu(), k.float().cpu(), v.float().cpu())
    got = out.cpu().numpy().astype(np.float64)
    err = np.abs(got - ref).max() / np.abs(ref).max()
    assert err <= TOL, err
    return err


@pytest.mark.parametrize("n", [1, 5, 15, 16, 17, 63, 64, 65, 127, 128, 129, 512, 640, 4097, 8191])
def test_attention_matches_oracle(n):
    step("attention n=%d" % n)
    q, k, v = synth.attention_inputs(n, "cuda", seed=30 + n % 11)
    out = tw.attention_decode(q, k, v)
    torch.cuda.synchronize()
    check(q, k, v, out)


@pytest.mark.parametrize("H,Hkv", [(8, 8), (16, 8), (64, 8), (2, 1)])
def test_attention_group_sizes(H, Hkv):
    step("attention H=%d Hkv=%d" % (H, Hkv))
    q, k, v = synth.attention_inputs(300, "cuda", seed=40, heads=H, kv_heads=Hkv)
    out = tw.attention_decode(q, k, v)
    torch.cuda.synchronize()
    check(q, k, v, out)


def test_attention_long_context():
    n = 131072      # the pages' maximum context, as one global layer's cache
    step("attention n=%d" % n)
    q, k, v = synth.attention_inputs(n, "cuda", seed=41)
    out = tw.attention_decode(q, k, v)
    torch.cuda.synchronize()
    check(q, k, v, out)


def test_attention_sharp_softmax_and_single_slot():
    step("attention sharp softmax")
    q, k, v = synth.attention_inputs(640, "cuda", seed=42)
    q8 = (q.float() * 8).to(torch.bfloat16)          # scores up to ~ +-60: a few slots dominate
    out = tw.attention_decode(q8, k, v)
    torch.cuda.synchronize()
    check(q8, k, v, out)
    q1, k1, v1 = synth.attention_inputs(1, "cuda", seed=43)
    out1 = tw.attention_decode(q1, k1, v1)
    torch.cuda.synchronize()
    # one slot: every query head returns its KV head's value row exactly
    assert torch.equal(out1, v1[0].float().repeat_interleave(4, dim=0))


def test_attention_window_ring_slot_order():
    # a windowed layer at position 900: its ring of 512 slots holds positions 388..899, position p
    # in slot p mod 512; the oracle attends over the same positions in position order
    step("attention ring")
    ctx, W = 900, synth.ATTN_WINDOW
    q, k, v = synth.attention_inputs(ctx, "cuda", seed=44)
    pos = torch.arange(ctx - W, ctx)
    slot_of = pos % W
    kr = torch.empty_like(k[:W])
    vr = torch.empty_like(v[:W])
    kr[slot_of.cuda()] = k[pos.cuda()]
    vr[slot_of.cuda()] = v[pos.cuda()]
    out = tw.attention_decode(q, kr, vr)
    torch.cuda.synchronize()
    check(q, k[ctx - W:], v[ctx - W:], out)


def test_attention_reuses_workspace_and_is_deterministic():
    step("attention determinism")
    q, k, v = synth.attention_inputs(640, "cuda", seed=45)
    ws = torch.empty(tw.attention_decode_workspace_bytes(16, 128, 4097), dtype=torch.uint8, device="cuda")
    a = tw.attention_decode(q, k, v, workspace=ws).clone()
    q2, k2, v2 = synth.attention_inputs(4097, "cuda", seed=46)
    c = tw.attention_decode(q2, k2, v2, workspace=ws).clone()
    b = tw.attention_decode(q, k, v, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    check(q2, k2, v2, c)


# ---- the one-launch form ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,H,Hkv", [(1, 16, 4), (15, 16, 4), (16, 16, 4), (17, 16, 4), (100, 8, 8),
                                     (512, 16, 4), (640, 16, 4), (1000, 16, 8), (1024, 2, 1),
                                     (333, 64, 8)])
def test_attention_one_launch_equals_two_launches(n, H, Hkv):
    # the same partials merged in the same order: the same bits as attention_decode, and within
    # the oracle tolerance; the workspace is zero-filled again after the call
    step("attention one launch n=%d H=%d Hkv=%d" % (n, H, Hkv))
    q, k, v = synth.attention_inputs(n, "cuda", seed=50 + n % 13, heads=H, kv_heads=Hkv)
    ws = tw.attention_decode_one_workspace(H, 128, n)
    one = tw.attention_decode_one(q, k, v, ws)
    two = tw.attention_decode(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(one, two)
    assert not torch.any(ws)
    check(q, k, v, one)


def test_attention_one_launch_reused_workspace():
    # calls of several sizes and group shapes on one workspace (sized for the largest), each
    # equal to attention_decode; between calls every word is zero again
    ws = tw.attention_decode_one_workspace(64, 128, 1024)
    for i, (n, H, Hkv) in enumerate([(1024, 64, 8), (640, 16, 4), (1, 16, 4), (1024, 16, 4),
                                     (37, 64, 8), (640, 16, 4)]):
        step("attention one launch, reused workspace, call %d (n=%d)" % (i, n))
        q, k, v = synth.attention_inputs(n, "cuda", seed=60 + i, heads=H, kv_heads=Hkv)
        one = tw.attention_decode_one(q, k, v, ws)
        two = tw.attention_decode(q, k, v)
        torch.cuda.synchronize()
        assert torch.equal(one, two), i
        assert not torch.any(ws), i


def test_attention_one_launch_sharp_softmax_and_rejects_long_caches():
    step("attention one launch, sharp softmax")
    q, k, v = synth.attention_inputs(640, "cuda", seed=42)
    q8 = (q.float() * 8).to(torch.bfloat16)
    ws = tw.attention_decode_one_workspace(16, 128, 640)
    out = tw.attention_decode_one(q8, k, v, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, tw.attention_decode(q8, k, v))
    check(q8, k, v, out)
    q2, k2, v2 = synth.attention_inputs(1025, "cuda", seed=43)
    with pytest.raises(RuntimeError):
        tw.attention_decode_one(q2, k2, v2, ws)
