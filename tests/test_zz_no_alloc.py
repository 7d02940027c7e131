"""ternary_moe_ffn_decode_static (the decode with the library's static per-device scratch, for
callers that cannot allocate) against ternary_moe_ffn_decode with a caller's workspace, through the
C ABI: bit for bit, on two calls in a row, the second with a smaller input, and the health word."""
import pytest
import torch

import synth
import ternary_weight_moe_amd as tw
from parity_util import require_gpu, step

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def gpu_layers(wl, n):
    out = []
    for l in range(n):
        w = synth.layer_weights(wl, l, device="cuda")
        out.append(tw.MoELayer.from_ternary(w["w_router"], w["t_gate"], w["t_up"], w["t_down"],
                                            w["s_gate"], w["s_up"], w["s_down"], top_k=wl.top_k,
                                            pre_rmsnorm=wl.pre_rmsnorm))
    return out


def same_bits(a, b):
    return torch.equal(a.view(torch.int16 if a.dtype == torch.bfloat16 else torch.int32),
                       b.view(torch.int16 if b.dtype == torch.bfloat16 else torch.int32))


def test_static_decode_equals_workspace_decode_on_two_calls():
    health = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    # call 1: eight full-size layers with the pre-RMSNorm (the one-launch stacked decode)
    step("static decode: 8 full-size stack layers")
    big = gpu_layers(synth.STACK24_B1, 8)
    x = synth.activations(synth.STACK24_B1, 1, device="cuda", seed=91)[0]
    got = tw.ternary_moe_ffn_decode_static(big, x, health=health)
    ref = tw.ternary_moe_ffn_decode(big, x)
    torch.cuda.synchronize()
    assert same_bits(got, ref) and int(health.item()) == 0
    # call 2, right after on the same scratch: a smaller input (the fp32 d_model 256 layer, served
    # by the per-layer kernels), then the first shape again
    step("static decode: small fp32 layer after the stack")
    small = gpu_layers(synth.SMALL_LAYER_B1, 1)
    xs = synth.activations(synth.SMALL_LAYER_B1, 3, device="cuda", seed=92)
    health.fill_(-1)
    for t in range(3):
        got = tw.ternary_moe_ffn_decode_static(small, xs[t], health=health)
        ref = tw.ternary_moe_ffn_decode(small, xs[t])
        torch.cuda.synchronize()
        assert same_bits(got, ref) and int(health.item()) == 0, t
    step("static decode: the stack again")
    got = tw.ternary_moe_ffn_decode_static(big[:3], x)
    ref = tw.ternary_moe_ffn_decode(big[:3], x)
    torch.cuda.synchronize()
    assert same_bits(got, ref)


def test_static_decode_in_a_graph():
    # captured and replayed (the caller allocates only the graph's input and output)
    step("static decode: captured in a graph")
    layers = gpu_layers(synth.MID_STACK_B1, 3)
    x = synth.activations(synth.MID_STACK_B1, 1, device="cuda", seed=93)[0]
    out = torch.empty_like(x)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        tw.ternary_moe_ffn_decode_static(layers, x, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        tw.ternary_moe_ffn_decode_static(layers, x, out=out)
    ref = tw.ternary_moe_ffn_decode(layers, x)
    torch.cuda.synchronize()
    for r in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert same_bits(out, ref), r
        tw.ternary_moe_ffn_decode(layers, x)   # eager work between the replays
        torch.cuda.synchronize()
