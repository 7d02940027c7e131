"""Helpers shared by the GPU parity tests: building the same seeded layer for the oracle and for the
HIP library, comparison rules and the near-tie rule for routing."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import synth
import ternary_weight_moe_amd as tw

# Near-tie tolerance for routing decisions (absolute, in logit units).  The GPU sums logits in fp32,
# the oracle in double; their difference is ~1e-6 on these workloads.
TAU = 1e-5


def step(msg: str):
    """Names the GPU step about to run (flushed, so a crash still shows which case it was)."""
    print("[gpu-step] " + msg, flush=True)
    sys.stdout.flush()


def require_gpu():
    import pytest
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X GPU")
    tw.lib()   # raises if the HIP library is not built: no fallback


def normwise(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.max(np.abs(b))
    return float(np.max(np.abs(a - b)) / den) if den > 0 else float(np.max(np.abs(a - b)))


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.numpy().astype(np.float64)


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


class LayerPair:
    """The same layer for the oracle (packed by the oracle) and for the GPU (packed by
    ternary_pack), from one draw of synth tensors."""

    def __init__(self, w: dict, top_k: int, pre_rmsnorm: bool, device="cuda"):
        gdev = torch.device(device)
        self.gpu = tw.MoELayer.from_ternary(w["w_router"].to(gdev), w["t_gate"], w["t_up"],
                                            w["t_down"], w["s_gate"], w["s_up"], w["s_down"],
                                            top_k=top_k, pre_rmsnorm=pre_rmsnorm)
        cpu = {k: v.cpu() for k, v in w.items()}
        self.ora = oracle.Layer(cpu["w_router"], cpu["t_gate"], cpu["t_up"], cpu["t_down"],
                                cpu["s_gate"], cpu["s_up"], cpu["s_down"],
                                pre_rmsnorm=pre_rmsnorm, top_k=top_k)
        torch.cuda.synchronize()
        assert int(self.gpu.bad_count.item()) == 0


def make_pair(workload, layer=0, device="cuda", seed=None, n_experts=None, pre=None, top_k=None):
    gen_dev = device if workload.d_model * workload.d_ff * (n_experts or workload.n_experts) > (1 << 22) else "cpu"
    w = synth.layer_weights(workload, layer, device=gen_dev, seed=seed, n_experts=n_experts)
    return LayerPair(w, top_k or workload.top_k, workload.pre_rmsnorm if pre is None else pre,
                     device)


def routing_alternatives(logits_row: np.ndarray, ids: np.ndarray, k: int, tau: float = TAU):
    """The oracle's routing plus, where its k-th and (k+1)-th logits lie within tau, the routing
    with those two exchanged; each with gates = softmax over the chosen logits."""
    out = [(ids.copy(), None)]
    order = np.lexsort((np.arange(len(logits_row)), -logits_row))
    if k < len(logits_row) and logits_row[order[k - 1]] - logits_row[order[k]] < tau:
        alt = ids.copy()
        alt[k - 1] = order[k]
        out.append((alt, None))
    res = []
    for sel, _ in out:
        l = logits_row[sel]
        e = np.exp(l - l[0])
        res.append((sel.astype(np.int32), e / e.sum()))
    return res


def check_routing(gpu_ids, gpu_gates, ora_logits, ora_ids, ora_gates, k, tau=TAU):
    """GPU routing must equal the oracle's, except across near-ties (< tau), where any selection and
    order consistent with the oracle's logits up to tau is accepted.  Returns #near-tie tokens."""
    ties = 0
    for t in range(gpu_ids.shape[0]):
        g = gpu_ids[t]
        l = ora_logits[t]
        if np.array_equal(g, ora_ids[t]):
            assert np.allclose(gpu_gates[t], ora_gates[t], rtol=1e-5, atol=1e-7), t
            continue
        ties += 1
        assert len(set(g.tolist())) == k
        rest = np.setdiff1d(np.arange(len(l)), g)
        if len(rest):
            assert l[g].min() >= l[rest].max() - tau, (t, g, ora_ids[t])
        assert np.all(l[g][:-1] >= l[g][1:] - tau), t
        ref = np.exp(l[g] - l[g][0])
        assert np.allclose(gpu_gates[t], ref / ref.sum(), rtol=1e-4), t
    return ties
