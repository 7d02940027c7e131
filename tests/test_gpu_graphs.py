"""Every call captured in a HIP graph (torch's graph capture of the library calls) and replayed
several times, with eager work and synchronisations between the replays: each replay must equal
the eager result bit for bit (the calls allocate nothing, record no memset, and keep no state
between calls other than their outputs)."""
import pytest
import torch

import synth
import ternary_weight_moe_amd as tw
from parity_util import require_gpu, step

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def replay_matches(fn, outs_of, reps=3):
    """fn() launches the call(s) into preallocated outputs; outs_of() returns them."""
    fn()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs_of()]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    for r in range(reps):
        for o in outs_of():
            o.fill_(-7)                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs_of(), ref):
            assert torch.equal(a, b), r


def test_graph_replay_ffn_decode_and_batched():
    step("graph: decode and batched FFN")
    wl = synth.SMALL_LAYER_B1
    w = synth.layer_weights(wl, 0, device="cuda")
    layer = tw.MoELayer.from_ternary(w["w_router"], w["t_gate"], w["t_up"], w["t_down"],
                                     w["s_gate"], w["s_up"], w["s_down"], top_k=wl.top_k)
    x1 = synth.activations(wl, 1, device="cuda")
    xb = synth.activations(wl, 37, device="cuda")
    o1 = torch.empty_like(x1[0])
    ob = torch.empty_like(xb)
    ws1 = torch.empty(tw.decode_workspace_bytes([layer]), dtype=torch.uint8, device="cuda")
    wsb = torch.empty(tw.batched_workspace_bytes(layer, 37, "float"), dtype=torch.uint8, device="cuda")

    # a full-size bf16 layer: the one-launch decode kernel
    wf = synth.layer_weights(synth.LAYER_B1, 0, device="cuda")
    lf = tw.MoELayer.from_ternary(wf["w_router"], wf["t_gate"], wf["t_up"], wf["t_down"],
                                  wf["s_gate"], wf["s_up"], wf["s_down"], top_k=synth.LAYER_B1.top_k)
    del wf
    xf = synth.activations(synth.LAYER_B1, 1, device="cuda")
    of = torch.empty_like(xf[0])
    wsf = torch.empty(tw.decode_workspace_bytes([lf, lf]), dtype=torch.uint8, device="cuda")

    def fn():
        tw.ternary_moe_ffn_decode([layer], x1[0], out=o1, workspace=ws1)
        tw.ternary_moe_ffn_batched(layer, xb, act="float", out=ob, workspace=wsb)
        tw.ternary_moe_ffn_decode([lf, lf], xf[0], out=of, workspace=wsf)
    replay_matches(fn, lambda: [o1, ob, of])


def test_graph_replay_gemv_attention_head():
    step("graph: gemv, attention, head")
    w = synth.trits((1000, 2048), "cuda", 80, 0, "gate")
    c3 = tw.ternary_pack3(w)
    sc = synth.uniform((1000,), 0.01, 0.1, "cuda", 80, 0, "s_gate").contiguous()
    xq = synth.int8_codes(2048, "cuda", 80)
    xs = torch.tensor([0.02], dtype=torch.float32, device="cuda")
    y = torch.empty(1000, dtype=torch.float32, device="cuda")
    q, k, v = synth.attention_inputs(640, "cuda", seed=81)
    ao = torch.empty((16, 128), dtype=torch.float32, device="cuda")
    aws = torch.empty(tw.attention_decode_workspace_bytes(16, 128, 640), dtype=torch.uint8, device="cuda")
    ao1 = torch.empty((16, 128), dtype=torch.float32, device="cuda")
    aws1 = tw.attention_decode_one_workspace(16, 128, 640)   # every replay leaves it zero-filled
    f = synth.head_inputs(300, 8, 1024, "cuda", seed=82)
    h = synth.head_hidden(1024, "cuda", seed=82)
    hws = torch.empty(tw.lib().flash_head_workspace_bytes(300), dtype=torch.uint8, device="cuda")
    res = {}

    def fn():
        tw.ternary_gemv_i8(c3, 3, sc, 2048, xq, xs, out=y)
        tw.attention_decode(q, k, v, out=ao, workspace=aws)
        tw.attention_decode_one(q, k, v, aws1, out=ao1)
        res["head"] = tw.flash_head(h, f["centroids"], f["centroid_scales"], f["w_clustered"],
                                    f["member_ids"], 40, workspace=hws)
    fn()
    torch.cuda.synchronize()
    sel, ids, lg = res["head"]
    ref = [y.clone(), ao.clone(), sel.clone(), ids.clone(), lg.clone(), ao1.clone()]
    assert torch.equal(ao1, ao)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    outs = [y, ao, *res["head"], ao1]       # the head's outputs allocated inside the capture
    for r in range(3):
        y.fill_(-7)
        ao.fill_(-7)
        ao1.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a, b), r
        assert not torch.any(aws1), r
