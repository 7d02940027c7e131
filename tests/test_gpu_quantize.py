"""ternary_quantize (float weights -> packed ternary codes + per-row scales, per-row absmean) on
the GPU through the C ABI, against the CPU oracle: bit-exact codes and scales (the scale decides
integer codes, so both sides follow the same fp32 order), at full layer size on sampled rows and
on whole matrices at a smaller size, on ragged, long, zero and tie rows, and fed into the FFN."""
import numpy as np
import pytest
import torch

import oracle
import synth
import ternary_weight_moe_amd as tw
from parity_util import normwise, require_gpu, step, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def check_rows(w_gpu: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, rows=None):
    """Bit-exact comparison of the GPU result with the oracle on the given rows (all by default)."""
    cols = w_gpu.shape[-1]
    w2 = w_gpu.reshape(-1, cols)
    p2 = packed.reshape(-1, cols // 4)
    s2 = scales.reshape(-1)
    if rows is not None:
        idx = torch.as_tensor(rows, device=w2.device)
        w2, p2, s2 = w2[idx], p2[idx], s2[idx]
    t_ref, s_ref = oracle.quantize_absmean(w2.cpu())
    p_ref, bad = oracle.pack(t_ref)
    assert bad == 0
    got_p, got_s = p2.cpu().numpy(), s2.cpu().numpy()
    assert np.array_equal(got_s.view(np.uint32), s_ref.view(np.uint32)), \
        int(np.sum(got_s.view(np.uint32) != s_ref.view(np.uint32)))
    assert np.array_equal(got_p, p_ref), int(np.sum(got_p != p_ref))


def test_quantize_full_layer_sampled_rows():
    wl = synth.QUANTIZE_LAYER
    step("quantize_layer: draw float expert weights on the GPU")
    w = synth.float_expert_weights(wl, 0, device="cuda")
    g = torch.Generator().manual_seed(5)
    for name in ("w_gate", "w_up", "w_down"):
        step("quantize_layer: %s %s" % (name, tuple(w[name].shape)))
        packed, scales = tw.ternary_quantize(w[name])
        torch.cuda.synchronize()
        n = w[name].numel() // w[name].shape[-1]
        rows = torch.cat([torch.tensor([0, 1, n - 2, n - 1]), torch.randint(0, n, (3000,), generator=g)])
        check_rows(w[name], packed, scales, rows.tolist())


@pytest.mark.parametrize("E", [8])
def test_quantize_whole_matrices(E):
    wl = synth.QUANTIZE_LAYER
    step("quantize: %d experts, every row" % E)
    w = synth.float_expert_weights(wl, 1, device="cuda", n_experts=E)
    for name in ("w_gate", "w_up", "w_down"):
        packed, scales = tw.ternary_quantize(w[name])
        torch.cuda.synchronize()
        check_rows(w[name], packed, scales)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("cols", [8, 40, 264, 512, 520, 2048, 4096, 6152])
def test_quantize_ragged_long_and_special_rows(dtype, cols):
    # up to 512 (64 chunks): four rows per wave, 40 and 264 with partly filled lanes; 520 = 65
    # chunks (a ragged last lane group), 4096 and 6152 (> 256 chunks: the two-pass form); 37 rows
    # leave the last wave's row groups partly empty
    step("quantize: %s cols %d" % (dtype, cols))
    g = torch.Generator().manual_seed(cols)
    w = (torch.randn((37, cols), generator=g) * 0.05)
    w[3] = 0.0                                   # zero row
    w[4] = 0.0
    w[4, cols - 1] = -2.5                        # a single nonzero, last element
    w[5] = 15.0
    w[5, 0] = 7.0                                # |w| / g = 0.5 exactly when cols == 8
    w[6] = torch.where(torch.rand(cols, generator=g) < 0.5, -0.125, 0.125)
    w[7] = torch.randint(-1, 2, (cols,), generator=g).float() * 0.03125
    w = w.to(dtype).cuda().contiguous()
    packed, scales = tw.ternary_quantize(w)
    torch.cuda.synchronize()
    check_rows(w, packed, scales)
    s = scales.cpu().numpy()
    assert s[3] == 0.0 and np.all(packed.cpu().numpy()[3] == 0)


def test_quantize_empty_is_a_no_op():
    w = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    packed, scales = tw.ternary_quantize(w)
    torch.cuda.synchronize()
    assert packed.numel() == 0 and scales.numel() == 0


def test_quantized_weights_feed_the_ffn():
    # float expert weights of the small layer -> ternary_quantize -> decode on the GPU, against the
    # oracle's FFN on the oracle's own quantisation of the same weights (equal codes and scales)
    wl = synth.SMALL_LAYER_B1
    step("quantize: small layer fed into the decode")
    fw = synth.float_expert_weights(wl, 0, dtype="f32", std=0.05)
    base = synth.layer_weights(wl, 0)
    gpu = tw.MoELayer.from_float(base["w_router"].cuda(), fw["w_gate"], fw["w_up"], fw["w_down"],
                                 top_k=wl.top_k)
    tq = {k: oracle.quantize_absmean(fw[k]) for k in ("w_gate", "w_up", "w_down")}
    ora = oracle.Layer(base["w_router"], tq["w_gate"][0], tq["w_up"][0], tq["w_down"][0],
                       tq["w_gate"][1], tq["w_up"][1], tq["w_down"][1], top_k=wl.top_k)
    x = synth.activations(wl, 4, seed=3)
    for t in range(4):
        out = tw.ternary_moe_ffn_decode([gpu], x[t].cuda())
        torch.cuda.synchronize()
        ref, _, _, _ = oracle.moe_layer(ora, x[t][None])
        assert normwise(to_np(out).astype(np.float64), ref[0]) <= 1e-4
