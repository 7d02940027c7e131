"""Algorithmic byte and operation counts for the ternary MoE FFN workloads (host-side, no GPU).

"Algorithmic" means what the method itself must move: every weight byte it touches, read once per
batch (packed codes, per-row scales, router), plus the activations in and out once.
Intermediates (logits, h, per-expert outputs) are not counted; extra traffic they cause shows up in
hardware counters instead.

The accounting follows the bandwidth argument of "A 20B AI Model Trained in Ternary Just Hit 218
Tokens/Second on a $599 Mac Mini" (section "What Ternary Actually Means"): bytes read per token
divided by the memory bandwidth bounds the decode rate, and the measured rate over that bound is
the fraction of peak bandwidth in use.
"""
from __future__ import annotations

HBM_PEAK_BPS = 8.0e12          # MI355X HBM3E, published peak
INT8_MFMA_PEAK_OPS = 5.0e15    # MI355X dense int8 MFMA, published peak (ops/s)


def _dt_bytes(dt: str) -> int:
    return {"f32": 4, "bf16": 2, "int8": 1}[dt]


def expert_bytes(d_model: int, d_ff: int) -> int:
    """Packed codes plus fp32 row scales of one expert (gate, up: [F][d/4]; down: [d][F/4])."""
    codes = 2 * d_ff * ((d_model + 3) // 4) + d_model * ((d_ff + 3) // 4)
    scales = 4 * (2 * d_ff + d_model)
    return codes + scales


def router_bytes(d_model: int, n_experts: int, router_dtype: str) -> int:
    return n_experts * d_model * _dt_bytes(router_dtype)


def layer_bytes(w, n_tokens: int = 1, distinct_experts: int | None = None) -> int:
    """Bytes one layer must move for n_tokens tokens when each touched expert is read once.
    For batch 1, distinct_experts = top_k."""
    D = w.top_k if distinct_experts is None else distinct_experts
    act = n_tokens * w.d_model * (_dt_bytes(w.io_dtype) + _dt_bytes(w.out_dtype))
    return D * expert_bytes(w.d_model, w.d_ff) + router_bytes(w.d_model, w.n_experts,
                                                              w.router_dtype) + act


def stack_bytes_per_token(w) -> int:
    """Batch-1 decode through w.n_layers layers: each layer reads its k experts and its router."""
    return w.n_layers * layer_bytes(w, 1)


def int8_ops(w, n_pairs: int) -> int:
    """Multiply-add operations (counted as 2 ops) of the ternary contractions for n_pairs
    (token, expert) pairs: gate + up ([F] x [d]) and down ([d] x [F])."""
    return n_pairs * 3 * w.d_model * w.d_ff * 2


def quantize_bytes(w) -> int:
    """Algorithmic HBM bytes of quantising one layer's float expert weights (gate, up, down) to
    packed ternary codes: every float read once, every code byte and per-row scale written once."""
    E, d, F = w.n_experts, w.d_model, w.d_ff
    n_w = 3 * E * F * d
    rows = 2 * E * F + E * d
    return n_w * _dt_bytes(w.router_dtype) + n_w // 4 + 4 * rows


def gemv_bytes(rows: int, cols: int, layout: int) -> int:
    """Algorithmic HBM bytes of one int8 ternary GEMV: every code byte and row scale read once,
    the int8 input and its scale read once, one fp32 output per row written."""
    row_bytes = cols // 4 if layout == 2 else ((cols + 4) // 5 + 15) // 16 * 16
    return rows * row_bytes + 4 * rows + cols + 4 + 4 * rows


def ceiling_rate(bytes_per_unit: float, bandwidth_bps: float) -> float:
    """Units per second at which the bytes alone saturate the bandwidth."""
    return bandwidth_bps / bytes_per_unit


def fraction_of_peak(rate: float, bytes_per_unit: float, bandwidth_bps: float) -> float:
    return rate * bytes_per_unit / bandwidth_bps
