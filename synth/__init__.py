"""Seeded synthetic inputs for the ternary MoE FFN workloads.

This module only draws random tensors of the shapes and distributions below; it holds none of the
method's arithmetic (no packing, routing, rounding beyond the dtype cast of a draw, or FFN math).
Both the oracle side and the HIP side of every test take their inputs from here.

Workloads (the pages give the model's shape -- 24 layers, 256 experts with 8 active -- in
"How a 20B Model Hits 120 tok/s on an iPhone" and in the section "The Architecture: Designed for
the Hardware" of "A 20B AI Model Trained in Ternary Just Hit 218 Tokens/Second on a $599 Mac
Mini"; the pages give no d_model or expert width, so those are fixed here):

  small_layer_b1   one layer, d=256, 16 experts, F=128, top-2, fp32 router and activations
  layer_b1         one layer, d=2048, 256 experts, F=512, top-8, bf16 router and activations
  stack24_b1       24 independently seeded layer_b1 layers with a pre-RMSNorm, batch 1
  batched_b64      one layer_b1 layer, 64 tokens (float and int8 activation variants)
  prefill_4096     one layer_b1 layer, 4096 tokens, int8 activations, fp32 output

Distributions: router ~ N(0, 0.02) (0.02 is the standard deviation); ternary weights iid uniform
over {-1, 0, +1}; per-row scales ~ U[0.01, 0.1] (continuous, fp32); activations ~ N(0, 1).
bf16 tensors are the round-to-nearest-even cast of the fp32 draw.  Every tensor has its own
torch.Generator keyed by (workload seed, layer, tensor kind, stream), so any tensor can be drawn
again on its own and the draw does not depend on which other tensors were drawn first.
The same key gives the same values on the same device type; CPU and GPU draws differ.
"""
from __future__ import annotations

import dataclasses

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    d_model: int
    n_experts: int
    d_ff: int
    top_k: int
    router_dtype: str      # "f32" or "bf16"
    io_dtype: str          # activation dtype in
    out_dtype: str         # output dtype
    batch: int = 1
    n_layers: int = 1
    pre_rmsnorm: bool = False
    act: str = "float"     # "float" or "int8"
    seed: int = 0
    steps: int = 1


SMALL_LAYER_B1 = Workload("small_layer_b1", 256, 16, 128, 2, "f32", "f32", "f32", seed=1000)
LAYER_B1 = Workload("layer_b1", 2048, 256, 512, 8, "bf16", "bf16", "bf16", seed=1001)
STACK24_B1 = Workload("stack24_b1", 2048, 256, 512, 8, "bf16", "bf16", "bf16", n_layers=24,
                      pre_rmsnorm=True, seed=1002, steps=256)
BATCHED_B64 = Workload("batched_b64", 2048, 256, 512, 8, "bf16", "bf16", "bf16", batch=64,
                       seed=1003)
BATCHED_B64_INT8 = dataclasses.replace(BATCHED_B64, name="batched_b64_int8", act="int8")
PREFILL_4096 = Workload("prefill_4096", 2048, 256, 512, 8, "bf16", "bf16", "f32", batch=4096,
                        act="int8", seed=1004)

# test-only shapes: a mid-size stack (a second shape of the one-launch stacked decode) and a
# narrow bf16 layer that the stacked decode does not serve (per-layer kernels)
MID_STACK_B1 = Workload("mid_stack_b1", 1024, 64, 256, 4, "bf16", "bf16", "bf16", n_layers=3,
                        pre_rmsnorm=True, seed=1005)
NARROW_LAYER_B1 = Workload("narrow_layer_b1", 512, 16, 128, 2, "bf16", "bf16", "bf16", seed=1006)

# float expert weights of one full-size layer, quantised to ternary (gate/up [E][F][d], down
# [E][d][F], bf16 ~ N(0, 0.02))
QUANTIZE_LAYER = Workload("quantize_layer", 2048, 256, 512, 8, "bf16", "bf16", "bf16", seed=1007)

WORKLOADS = {w.name: w for w in (SMALL_LAYER_B1, LAYER_B1, STACK24_B1, BATCHED_B64,
                                 BATCHED_B64_INT8, PREFILL_4096, MID_STACK_B1, NARROW_LAYER_B1,
                                 QUANTIZE_LAYER)}

_KINDS = {"router": 1, "gate": 2, "up": 3, "down": 4, "s_gate": 5, "s_up": 6, "s_down": 7,
          "x": 8, "fgate": 9, "fup": 10, "fdown": 11, "xq": 12, "q": 13, "k": 14, "v": 15,
          "head": 16, "perm": 17, "h": 18}

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _gen(device, seed: int, layer: int, kind: str, stream: int = 0) -> torch.Generator:
    key = (seed * 1_000_003 + layer * 10_007 + _KINDS[kind] * 101 + stream) & ((1 << 62) - 1)
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(key)
    return g


def trits(shape, device, seed, layer, kind) -> torch.Tensor:
    """int8 values iid uniform over {-1, 0, +1}."""
    g = _gen(device, seed, layer, kind)
    return torch.randint(-1, 2, tuple(shape), dtype=torch.int8, device=device, generator=g)


def normal(shape, std, dtype, device, seed, layer, kind, stream=0) -> torch.Tensor:
    g = _gen(device, seed, layer, kind, stream)
    v = torch.randn(tuple(shape), dtype=torch.float32, device=device, generator=g)
    if std != 1.0:
        v = v * std
    return v.to(dtype)


def uniform(shape, lo, hi, device, seed, layer, kind) -> torch.Tensor:
    g = _gen(device, seed, layer, kind)
    return torch.rand(tuple(shape), dtype=torch.float32, device=device, generator=g) * (hi - lo) + lo


def layer_weights(w: Workload, layer: int = 0, device="cpu", seed: int | None = None,
                  n_experts: int | None = None) -> dict:
    """Unpacked weights of one layer: router [E][d], ternary int8 t_gate/t_up [E][F][d],
    t_down [E][d][F], fp32 scales s_gate/s_up [E][F], s_down [E][d]."""
    s = w.seed if seed is None else seed
    E = w.n_experts if n_experts is None else n_experts
    d, F = w.d_model, w.d_ff
    return dict(
        w_router=normal((E, d), 0.02, _DT[w.router_dtype], device, s, layer, "router"),
        t_gate=trits((E, F, d), device, s, layer, "gate"),
        t_up=trits((E, F, d), device, s, layer, "up"),
        t_down=trits((E, d, F), device, s, layer, "down"),
        s_gate=uniform((E, F), 0.01, 0.1, device, s, layer, "s_gate"),
        s_up=uniform((E, F), 0.01, 0.1, device, s, layer, "s_up"),
        s_down=uniform((E, d), 0.01, 0.1, device, s, layer, "s_down"),
    )


def float_expert_weights(w: Workload, layer: int = 0, device="cpu", seed: int | None = None,
                         n_experts: int | None = None, dtype: str | None = None,
                         std: float = 0.02) -> dict:
    """Float (not yet ternary) expert weights of one layer: w_gate, w_up [E][F][d] and w_down
    [E][d][F] ~ N(0, std) in the workload's router dtype (or `dtype`)."""
    s = w.seed if seed is None else seed
    E = w.n_experts if n_experts is None else n_experts
    d, F = w.d_model, w.d_ff
    dt = _DT[dtype or w.router_dtype]
    return dict(
        w_gate=normal((E, F, d), std, dt, device, s, layer, "fgate"),
        w_up=normal((E, F, d), std, dt, device, s, layer, "fup"),
        w_down=normal((E, d, F), std, dt, device, s, layer, "fdown"),
    )


def activations(w: Workload, n_tokens: int | None = None, device="cpu", seed: int | None = None,
                stream: int = 0) -> torch.Tensor:
    """x [T][d] ~ N(0, 1) in the workload's input dtype."""
    s = w.seed if seed is None else seed
    T = w.batch if n_tokens is None else n_tokens
    return normal((T, w.d_model), 1.0, _DT[w.io_dtype], device, s, 0, "x", stream)


def int8_codes(n: int, device="cpu", seed: int = 11, stream: int = 0) -> torch.Tensor:
    """n int8 activation codes iid uniform over [-127, 127] (the range of absmax quantisation)."""
    g = _gen(device, seed, 0, "xq", stream)
    return torch.randint(-127, 128, (n,), dtype=torch.int8, device=device, generator=g)


# ternary GEMV over the gate and up rows of one full-size layer's 256 experts (2 x 256 x 512 rows
# of 2048 weights): 128 MiB of 2-bit codes, 104 MiB in base 3
GEMV_ROWS, GEMV_COLS = 2 * 256 * 512, 2048


# decode attention: 16 query heads over 4 KV heads of 128 (16 x 128 = d_model 2048); the pages'
# 640-token benchmark context for the 6 global layers, a 512-slot ring for the 18 windowed ones
ATTN_HEADS, ATTN_KV_HEADS, ATTN_HEAD_DIM = 16, 4, 128
ATTN_CONTEXT, ATTN_WINDOW, ATTN_GLOBAL_LAYERS, ATTN_WINDOW_LAYERS = 640, 512, 6, 18


def attention_inputs(n_slots: int, device="cpu", seed: int = 21, layer: int = 0,
                     heads: int = ATTN_HEADS, kv_heads: int = ATTN_KV_HEADS,
                     head_dim: int = ATTN_HEAD_DIM) -> tuple:
    """q [heads][head_dim], k and v [n_slots][kv_heads][head_dim], all N(0, 1) in bf16."""
    q = normal((heads, head_dim), 1.0, torch.bfloat16, device, seed, layer, "q")
    k = normal((n_slots, kv_heads, head_dim), 1.0, torch.bfloat16, device, seed, layer, "k")
    v = normal((n_slots, kv_heads, head_dim), 1.0, torch.bfloat16, device, seed, layer, "v")
    return q, k, v


# approximate output head: 151,936 tokens in 4,748 clusters of 32 (the pages: about 151,000 tokens
# in 4,748 clusters), hidden size 2048, the top 512 clusters
HEAD_CLUSTERS, HEAD_CLUSTER_SIZE, HEAD_TOP, HEAD_D = 4748, 32, 512, 2048


def head_inputs(n_clusters: int = HEAD_CLUSTERS, cluster_size: int = HEAD_CLUSTER_SIZE,
                d: int = HEAD_D, device="cpu", seed: int = 23) -> dict:
    """Head rows w_clustered [ncl][cs][d] ~ N(0, 0.02) bf16 in cluster-major order, member_ids
    [ncl][cs] a random permutation of the token ids, centroids [ncl][d/2] uint8 with every nibble
    iid uniform over 0..15 (values -8..7 in offset binary), centroid scales U[0.01, 0.1] fp32."""
    w = normal((n_clusters, cluster_size, d), 0.02, torch.bfloat16, device, seed, 0, "head")
    g = _gen(device, seed, 0, "perm")
    members = torch.randperm(n_clusters * cluster_size, generator=g, device=device)
    members = members.to(torch.int32).reshape(n_clusters, cluster_size).contiguous()
    gc = _gen(device, seed, 1, "perm")
    cent = torch.randint(0, 256, (n_clusters, d // 2), generator=gc, device=device).to(torch.uint8)
    scales = uniform((n_clusters,), 0.01, 0.1, device, seed, 1, "head").contiguous()
    return dict(w_clustered=w.contiguous(), member_ids=members, centroids=cent.contiguous(),
                centroid_scales=scales)


def head_hidden(d: int = HEAD_D, device="cpu", seed: int = 23, stream: int = 0) -> torch.Tensor:
    """A hidden state h [d] ~ N(0, 1) bf16."""
    return normal((d,), 1.0, torch.bfloat16, device, seed, 0, "h", stream)


def routing(n_tokens: int, n_experts: int, top_k: int, device="cpu", seed: int = 7) -> tuple:
    """A synthetic routing for tests that pass routing in: per token, top_k distinct experts in
    random order and positive gates drawn U[0.01, 1] (not normalised)."""
    g = _gen(device, seed, 0, "x", 99)
    keys = torch.rand((n_tokens, n_experts), generator=g, device=device)
    ids = keys.argsort(dim=1)[:, :top_k].to(torch.int32).contiguous()
    gates = torch.rand((n_tokens, top_k), generator=g, device=device) * 0.99 + 0.01
    return ids, gates.contiguous()
