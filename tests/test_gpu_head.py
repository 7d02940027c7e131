"""Approximate output head on the GPU through the C ABI, against the CPU oracle: the selected
clusters and token ids exactly (the scores are exact integer sums scaled by the same two fp32
roundings, so both sides rank identically), the logits within a bound derived from fp32 summation:
|logit - exact| <= 2^-22 * d * sum_i |w_i h_i| (d products, each partial sum rounding at most
2^-24 relative; the factor 4 covers the lane partials and the wave tree)."""
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


def check_logits(f, h, sel, ids, logits, rows=None):
    w = f["w_clustered"]
    s = sel.cpu().numpy()
    lg = logits.cpu().numpy().astype(np.float64)
    hv = h.float().cpu().numpy().astype(np.float64)
    d = hv.size
    idx = [(j, m) for j in range(len(s)) for m in range(lg.shape[1])] if rows is None else rows
    W = w[torch.as_tensor([s[j] for j, _ in idx], device=w.device),
          torch.as_tensor([m for _, m in idx], device=w.device)].float().cpu().numpy().astype(np.float64)
    exact = W @ hv                                  # the oracle's logits are this product (pinned)
    bound = 2.0 ** -22 * d * (np.abs(W) @ np.abs(hv)) + 1e-30
    got = np.array([lg[j, m] for j, m in idx])
    assert np.all(np.abs(got - exact) <= bound), float(np.max(np.abs(got - exact) / bound))


@pytest.mark.parametrize("d,ncl,cs,top", [(512, 100, 8, 10), (1024, 37, 3, 37), (2048, 1000, 32, 512),
                                          (4096, 300, 16, 64), (2048, 1, 32, 1), (512, 1500, 2, 1024),
                                          (512, 3000, 2, 2000), (512, 8192, 1, 8192)])
def test_flash_head_matches_oracle(d, ncl, cs, top):
    step("flash_head d=%d ncl=%d cs=%d top=%d" % (d, ncl, cs, top))
    f = synth.head_inputs(ncl, cs, d, "cuda", seed=50 + ncl % 7)
    h = synth.head_hidden(d, "cuda", seed=50)
    sel, ids, logits = tw.flash_head(h, f["centroids"], f["centroid_scales"], f["w_clustered"],
                                     f["member_ids"], top)
    torch.cuda.synchronize()
    rsel, rids, rlg, _ = oracle.flash_head(h.float().cpu(), f["centroids"].cpu(),
                                           f["centroid_scales"].cpu(), f["w_clustered"].float().cpu(),
                                           f["member_ids"].cpu(), top)
    assert np.array_equal(sel.cpu().numpy(), rsel)
    assert np.array_equal(ids.cpu().numpy(), rids)
    bound = 2.0 ** -22 * d * np.abs(f["w_clustered"].float().cpu().numpy()[rsel]) @ np.abs(h.float().cpu().numpy())
    assert np.all(np.abs(logits.cpu().numpy() - rlg) <= bound + 1e-30)


def test_flash_head_ties_go_to_the_lower_cluster():
    step("flash_head ties")
    f = synth.head_inputs(64, 4, 512, "cuda", seed=60)
    f["centroids"][40] = f["centroids"][9]
    f["centroid_scales"][40] = f["centroid_scales"][9]
    f["centroids"][9:10] = 0x77              # values -1 everywhere: tie both at a known score
    f["centroids"][40:41] = 0x77
    h = synth.head_hidden(512, "cuda", seed=60)
    sel, ids, logits = tw.flash_head(h, f["centroids"], f["centroid_scales"], f["w_clustered"],
                                     f["member_ids"], 64)
    torch.cuda.synchronize()
    s = sel.cpu().numpy().tolist()
    assert sorted(s) == list(range(64)) and s.index(9) < s.index(40)
    rsel = oracle.flash_head(h.float().cpu(), f["centroids"].cpu(), f["centroid_scales"].cpu(),
                             f["w_clustered"].float().cpu(), f["member_ids"].cpu(), 64)[0]
    assert np.array_equal(sel.cpu().numpy(), rsel)


def test_flash_head_full_size():
    # the pages' sizes: 151,936 tokens in 4,748 clusters of 32, the top 512; selection checked
    # against the oracle's scores (cluster rows replaced by one zero row each, which the scores do
    # not read), logits on sampled rows
    ncl, cs, d, top = synth.HEAD_CLUSTERS, synth.HEAD_CLUSTER_SIZE, synth.HEAD_D, synth.HEAD_TOP
    step("flash_head full size")
    f = synth.head_inputs(ncl, cs, d, "cuda", seed=70)
    h = synth.head_hidden(d, "cuda", seed=70)
    sel, ids, logits = tw.flash_head(h, f["centroids"], f["centroid_scales"], f["w_clustered"],
                                     f["member_ids"], top)
    torch.cuda.synchronize()
    rsel = oracle.flash_head(h.float().cpu(), f["centroids"].cpu(), f["centroid_scales"].cpu(),
                             np.zeros((ncl, 1, d), np.float32), np.zeros((ncl, 1), np.int32), top)[0]
    assert np.array_equal(sel.cpu().numpy(), rsel)
    assert np.array_equal(ids.cpu().numpy(), f["member_ids"].cpu().numpy()[rsel])
    # every logit against the oracle's: the oracle reads only the rows of the clusters it selects,
    # so the others are left zero in its (double) copy of the head
    step("flash_head full size: oracle logits of the selected clusters")
    wv = np.zeros((ncl, cs, d), np.float64)
    idx = torch.as_tensor(rsel, device=f["w_clustered"].device, dtype=torch.int64)
    wv[rsel] = f["w_clustered"][idx].float().cpu().numpy()
    o = oracle.flash_head(h.float().cpu(), f["centroids"].cpu(), f["centroid_scales"].cpu(), wv,
                          f["member_ids"].cpu(), top)
    assert np.array_equal(o[0], rsel) and np.array_equal(ids.cpu().numpy(), o[1])
    bound = 2.0 ** -22 * d * (np.abs(wv[rsel]) @ np.abs(h.float().cpu().numpy().astype(np.float64)))
    assert np.all(np.abs(logits.cpu().numpy().astype(np.float64) - o[2]) <= bound + 1e-30)


def test_flash_head_tie_group_split_by_top():
    # 3000 clusters, all of one score except six above it; top = 1500 falls inside the tie group,
    # whose members span three 1024-id rows: the six first (by score), then the lowest 1494 tied ids
    # in ascending order
    step("flash_head tie group split by top")
    ncl, cs, d, top = 3000, 2, 512, 1500
    f = synth.head_inputs(ncl, cs, d, "cuda", seed=61)
    h = synth.head_hidden(d, "cuda", seed=61)
    # one centroid for all, of value +7 where h >= 0 and -8 elsewhere: a positive score
    nib = torch.where(h.float().cpu() >= 0, 15, 0).to(torch.uint8)
    row = (nib[0::2] | (nib[1::2] << 4)).to(torch.uint8)
    f["centroids"][:] = row.cuda()
    f["centroid_scales"][:] = f["centroid_scales"][0]
    high = [2999, 17, 1024, 2048, 5, 1500]
    for r, c in enumerate(high):
        f["centroid_scales"][c] = f["centroid_scales"][0] * (2.0 + r)
    sel, ids, logits = tw.flash_head(h, f["centroids"], f["centroid_scales"], f["w_clustered"],
                                     f["member_ids"], top)
    torch.cuda.synchronize()
    rsel, rids, rlg, sc = oracle.flash_head(h.float().cpu(), f["centroids"].cpu(),
                                            f["centroid_scales"].cpu(),
                                            f["w_clustered"].float().cpu(), f["member_ids"].cpu(), top)
    got = sel.cpu().numpy()
    assert np.array_equal(got, rsel) and np.array_equal(ids.cpu().numpy(), rids)
    # the expected order, independently of both: the high clusters by score (and id on ties),
    # then the rest of the ids ascending
    hi = sorted(high, key=lambda c: (-float(sc[c]), c))
    assert sc[0] > 0 and sc[hi[-1]] > sc[0]
    rest = [c for c in range(ncl) if c not in high][:top - len(high)]
    assert got.tolist() == hi + rest
