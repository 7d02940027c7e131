"""Base-3 packing (five ternary weights per byte) and the int8 ternary GEMV on the GPU through the
C ABI, against the CPU oracle: packed bytes bit-exact, GEMV outputs bit-exact (exact integer sums,
then the same two fp32 roundings) for both packed layouts, on ragged and full-size shapes."""
import numpy as np
import pytest
import torch

import oracle
import synth
import ternary_weight_moe_amd as tw
from parity_util import require_gpu, step

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def weights(rows, cols, seed):
    return synth.trits((rows, cols), "cuda", seed, 0, "gate")


def scales(rows, seed):
    return synth.uniform((rows,), 0.01, 0.1, "cuda", seed, 0, "s_gate").contiguous()


def bits(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


@pytest.mark.parametrize("rows,cols", [(1, 1), (3, 5), (5, 7), (17, 2048), (1000, 2051),
                                       (4096, 512), (2, 5120)])
def test_pack3_bit_exact(rows, cols):
    step("pack3 %dx%d" % (rows, cols))
    w = weights(rows, cols, 31)
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    p = tw.ternary_pack3(w, bad_count=bad)
    torch.cuda.synchronize()
    rb = tw.ternary_pack3_row_bytes(cols)
    ref, nbad = oracle.pack3(w.cpu(), rb)
    assert p.shape == (rows, rb) and nbad == 0 and int(bad.item()) == 0
    assert np.array_equal(p.cpu().numpy(), ref)


def test_pack3_counts_invalid_values():
    step("pack3 invalid values")
    w = weights(64, 100, 32)
    w[3, 7] = 2
    w[10, 99] = -128
    w[63, 0] = 5
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    p = tw.ternary_pack3(w, bad_count=bad)
    torch.cuda.synchronize()
    ref, nbad = oracle.pack3(w.cpu(), tw.ternary_pack3_row_bytes(100))
    assert nbad == 3 and int(bad.item()) == 3
    assert np.array_equal(p.cpu().numpy(), ref)


def run_gemv(layout, rows, cols, seed, wmat=None, xq=None):
    w = weights(rows, cols, seed) if wmat is None else wmat
    codes = tw.ternary_pack3(w) if layout == 3 else tw.ternary_pack(w)
    s = scales(rows, seed)
    x = synth.int8_codes(cols, "cuda", seed) if xq is None else xq
    xs = torch.tensor([0.0123], dtype=torch.float32, device="cuda")
    y = tw.ternary_gemv_i8(codes, layout, s, cols, x, xs)
    torch.cuda.synchronize()
    return w, s, x, xs, y


@pytest.mark.parametrize("layout,rows,cols", [
    (3, 1, 5), (3, 7, 13), (3, 1000, 2048), (3, 4099, 2051), (3, 300, 5120), (3, 65, 81),
    (3, 33, 512), (2, 1, 64), (2, 7, 192), (2, 1000, 2048), (2, 4099, 512), (2, 300, 4096)])
def test_gemv_i8_bit_exact(layout, rows, cols):
    step("gemv_i8 layout %d %dx%d" % (layout, rows, cols))
    w, s, x, xs, y = run_gemv(layout, rows, cols, 40 + rows % 7)
    ref = oracle.gemv_i8(w.cpu(), s.cpu(), x.cpu(), float(xs.item()))
    assert np.array_equal(bits(y.cpu().numpy()), bits(ref)), \
        int(np.sum(bits(y.cpu().numpy()) != bits(ref)))


def test_gemv_i8_layouts_agree_and_zero_input():
    step("gemv_i8 both layouts, zero input")
    rows, cols = 2000, 2048
    w = weights(rows, cols, 50)
    _, _, _, _, y2 = run_gemv(2, rows, cols, 50, wmat=w)
    _, _, _, _, y3 = run_gemv(3, rows, cols, 50, wmat=w)
    assert np.array_equal(bits(y2.cpu().numpy()), bits(y3.cpu().numpy()))
    z = torch.zeros(cols, dtype=torch.int8, device="cuda")
    _, _, _, _, y0 = run_gemv(3, rows, cols, 50, wmat=w, xq=z)
    assert not y0.cpu().numpy().any()
    # extreme activations: every input -127 against rows of all +1 (the largest |sum|)
    ones = torch.ones((3, 5120), dtype=torch.int8, device="cuda")
    full = torch.full((5120,), -127, dtype=torch.int8, device="cuda")
    w1, s1, x1, xs1, y1 = run_gemv(3, 3, 5120, 51, wmat=ones, xq=full)
    ref = oracle.gemv_i8(w1.cpu(), s1.cpu(), x1.cpu(), float(xs1.item()))
    assert np.array_equal(bits(y1.cpu().numpy()), bits(ref))


def test_gemv_i8_bytes_above_242_contribute_nothing():
    # bytes the packer never writes: the oracle's unpack reads them as five zeros
    step("gemv_i8 invalid base-3 bytes")
    rows, cols = 64, 2048
    w = weights(rows, cols, 52)
    codes = tw.ternary_pack3(w)
    codes[::3, 5::37] = 250
    codes[1, 0] = 243
    s = scales(rows, 52)
    x = synth.int8_codes(cols, "cuda", 52)
    xs = torch.tensor([0.5], dtype=torch.float32, device="cuda")
    y = tw.ternary_gemv_i8(codes, 3, s, cols, x, xs)
    torch.cuda.synchronize()
    wu, nbad = oracle.unpack3(codes.cpu(), cols)
    assert nbad > 0
    ref = oracle.gemv_i8(wu, s.cpu(), x.cpu(), 0.5)
    assert np.array_equal(bits(y.cpu().numpy()), bits(ref))


@pytest.mark.parametrize("layout", [2, 3])
def test_gemv_i8_full_size_sampled_rows(layout):
    # the benchmark's shape: the gate and up rows of one layer's 256 experts, 2048 inputs each
    rows, cols = synth.GEMV_ROWS, synth.GEMV_COLS
    step("gemv_i8 layout %d full size %dx%d" % (layout, rows, cols))
    w, s, x, xs, y = run_gemv(layout, rows, cols, 60)
    idx = torch.cat([torch.arange(0, 64), torch.randint(0, rows, (4000,), generator=torch.Generator().manual_seed(5)),
                     torch.arange(rows - 64, rows)]).cuda()
    ref = oracle.gemv_i8(w[idx].cpu(), s[idx].cpu(), x.cpu(), float(xs.item()))
    assert np.array_equal(bits(y[idx].cpu().numpy()), bits(ref))
