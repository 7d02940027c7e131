"""ternary_quantize (float weights -> packed ternary codes + per-row scales, per-row absmean) on
the GPU through the C ABI, against the CPU oracle's plain absmean (the mean of |w| rounded once to
fp32), at full layer size on sampled rows and on whole matrices at a smaller size, on ragged, long,
zero and tie rows, and fed into the FFN.

The pages fix no summation order for the mean, and the kernel sums |w| in its own fixed fp32 order,
so the two scales may differ by the rounding of an fp32 sum: at most (cols + 2) 2^-24 relative (any
order of cols nonnegative terms, one division, and the oracle's single rounding).  A code can then
differ only for a weight whose |w| lies within that window around half the scale, where either code
is a correct reading; those are counted and capped, every other code must be equal.  The kernel's
own order is checked as a determinism property, GPU against GPU, across launch shapes."""
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


def codes_of(packed: np.ndarray, cols: int) -> np.ndarray:
    """Trits of 2-bit packed rows (00 -> 0, 01 -> +1, 10 -> -1), weight 4b+j in bits 2j..2j+1."""
    p = packed.astype(np.uint8)
    c = np.stack([(p >> (2 * j)) & 3 for j in range(4)], axis=-1).reshape(p.shape[0], -1)[:, :cols]
    return np.where(c == 1, 1, np.where(c == 2, -1, 0)).astype(np.int8)


def check_rows(w_gpu: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, rows=None) -> int:
    """The GPU result against the oracle on the given rows (all by default); returns the number of
    codes that differ inside the rounding window (every other code must be equal)."""
    cols = w_gpu.shape[-1]
    w2 = w_gpu.reshape(-1, cols)
    p2 = packed.reshape(-1, cols // 4)
    s2 = scales.reshape(-1)
    if rows is not None:
        idx = torch.as_tensor(rows, device=w2.device)
        w2, p2, s2 = w2[idx], p2[idx], s2[idx]
    wf = w2.float().cpu().numpy()
    t_ref, s_ref = oracle.quantize_absmean(wf)
    got_t, got_s = codes_of(p2.cpu().numpy(), cols), s2.cpu().numpy()
    eps = (cols + 2) * 2.0 ** -24
    sr, sg = s_ref.astype(np.float64), got_s.astype(np.float64)
    assert np.array_equal(sr == 0, sg == 0)
    bad_s = np.abs(sg - sr) > eps * sr
    assert not bad_s.any(), (int(bad_s.sum()), float(np.max(np.abs(sg - sr) / np.maximum(sr, 1e-300))))
    diff = got_t != t_ref
    if diff.any():
        r, c = np.nonzero(diff)
        half = sr[r] / 2
        inside = np.abs(np.abs(wf[r, c].astype(np.float64)) - half) <= eps * half
        assert inside.all(), "codes differ outside the rounding window: %d" % int((~inside).sum())
    return int(diff.sum())


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
        nd = check_rows(w[name], packed, scales, rows.tolist())
        print("codes inside the rounding window that differ: %d of %d" % (nd, 3004 * w[name].shape[-1]))
        assert nd <= 8


@pytest.mark.parametrize("E", [8])
def test_quantize_whole_matrices(E):
    wl = synth.QUANTIZE_LAYER
    step("quantize: %d experts, every row" % E)
    w = synth.float_expert_weights(wl, 1, device="cuda", n_experts=E)
    for name in ("w_gate", "w_up", "w_down"):
        packed, scales = tw.ternary_quantize(w[name])
        torch.cuda.synchronize()
        nd = check_rows(w[name], packed, scales)
        print("codes inside the rounding window that differ: %d of %d" % (nd, w[name].numel()))
        assert nd <= 8


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
    assert check_rows(w, packed, scales) <= 2
    s = scales.cpu().numpy()
    assert s[3] == 0.0 and np.all(packed.cpu().numpy()[3] == 0)
    # rows whose |w| sum is exact in any order (all equal magnitudes, a single nonzero, trits times
    # a power of two) give the same scale on both sides, so every code is equal there
    t_ref, s_ref = oracle.quantize_absmean(w[3:8].float().cpu().numpy())
    assert np.array_equal(codes_of(packed[3:8].cpu().numpy(), cols), t_ref)
    assert np.array_equal(s[3:8], s_ref)


@pytest.mark.parametrize("cols", [264, 2048])
def test_quantize_is_deterministic_across_launch_shapes(cols):
    # the kernel's fixed fp32 order: a row gives the same bits whichever workgroup, wave or lane
    # group serves it -- whole matrix, rows permuted, and slices with odd offsets and counts
    step("quantize: determinism across launch shapes, cols %d" % cols)
    g = torch.Generator().manual_seed(77 + cols)
    w = (torch.randn((301, cols), generator=g) * 0.02).to(torch.bfloat16).cuda()
    p0, s0 = tw.ternary_quantize(w)
    perm = torch.randperm(301, generator=g).cuda()
    p1, s1 = tw.ternary_quantize(w[perm].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(p1, p0[perm]) and torch.equal(s1.view(torch.int32), s0[perm].view(torch.int32))
    for a, b in ((1, 2), (3, 40), (7, 300), (100, 301)):
        p2, s2 = tw.ternary_quantize(w[a:b].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(p2, p0[a:b]) and torch.equal(s2.view(torch.int32), s0[a:b].view(torch.int32))


def test_quantize_empty_is_a_no_op():
    w = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    packed, scales = tw.ternary_quantize(w)
    torch.cuda.synchronize()
    assert packed.numel() == 0 and scales.numel() == 0


def test_quantized_weights_feed_the_ffn():
    # float expert weights of the small layer -> ternary_quantize -> decode on the GPU, against the
    # oracle's FFN on the oracle's own quantisation of the same weights.  The weights are multiples
    # of 2^-16 below 1 in magnitude, so every sum of |w| over a row (at most 256 of them) is exact
    # in fp32 in any order: both sides find the same scales and therefore the same codes
    wl = synth.SMALL_LAYER_B1
    step("quantize: small layer fed into the decode")
    fw = synth.float_expert_weights(wl, 0, dtype="f32", std=0.05)
    fw = {k: (torch.round(v * 65536.0).clamp(-65535, 65535) / 65536.0) for k, v in fw.items()}
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
