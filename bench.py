#!/usr/bin/env python3
"""Benchmark of the ternary MoE FFN hot path on one MI355X.

Default workload (stack24_b1): batch-1 decode through 24 stacked ternary MoE FFN layers
(d_model 2048, 256 experts, expert width 512, top-8, pre-RMSNorm, residual between layers,
attention replaced by identity), steps chained (step t+1 decodes step t's output).  A step is one
token through all 24 layers.  Graphs of min(--steps, 256) consecutive steps are captured and
replayed at least 20 times in the timed region (each replay a sample; the steps actually timed are
reported).  The decode health word is checked after the timed replays, and one more replay must
equal the same steps run eagerly from the same state, bit for bit.

Prints ONE JSON line: tokens/s of the whole job, the roofline view of the step (algorithmic HBM
bytes per step / measured time per step against the 8 TB/s HBM peak) and the CPU oracle's rate on a
bounded sample of the same workload.

Other workloads (--workload): layer_b1 (one layer, batch 1), batched_b64 / batched_b64_int8 (one
layer, 64 tokens grouped by expert), prefill_4096 (one layer, 4096 tokens, int8 activations, routing
passed in; reported as int8 MFMA throughput), quantize_layer (float expert weights of one layer to
packed ternary codes and per-row scales); single-layer workloads rotate 8 independently seeded
layer copies so that the 256 MB last-level cache never holds the layer being timed.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import torch  # noqa: E402

import synth  # noqa: E402
import ternary_weight_moe_amd as tw  # noqa: E402
from ternary_weight_moe_amd import accounting  # noqa: E402

METRIC = "decode tok/s, 24-layer ternary MoE FFN stack, B=1; achieved HBM GB/s vs peak"
# sources of the kernel whose traffic counters are committed (the one-launch stacked decode)
# the sources of the dominant kernel of each workload that has committed counter runs
# (profiles/traffic_<workload>.json): the counters stand only while these are unchanged
KERNEL_SRCS = {w: [os.path.join(ROOT, "ternary_weight_moe_amd", "csrc", f) for f in fs] for w, fs in {
    "stack24_b1": ("tw_persist.hip", "tw_device.h", "tw_internal.h"),
    "prefill_4096": ("tw_prefill.hip", "tw_device.h", "tw_internal.h"),
}.items()}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash(workload: str = "stack24_b1") -> str:
    h = hashlib.sha256()
    for f in KERNEL_SRCS[workload]:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str):
    """HBM bytes per step from committed rocprofv3 counter runs, if they were taken on the current
    kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if workload not in KERNEL_SRCS or d.get("kernel_sha256_16") != kernel_hash(workload):
        return None
    return d.get("hbm_bytes_per_step")


def build_layer(wl, l, device="cuda", keep_cpu=False, pre=None):
    w = synth.layer_weights(wl, l, device=device)
    layer = tw.MoELayer.from_ternary(w["w_router"], w["t_gate"], w["t_up"], w["t_down"],
                                     w["s_gate"], w["s_up"], w["s_down"], top_k=wl.top_k,
                                     pre_rmsnorm=wl.pre_rmsnorm if pre is None else pre)
    cpu = {k: v.cpu() for k, v in w.items()} if keep_cpu else None
    del w
    return layer, cpu


def side_warmup(step_fn):
    """Two eager steps on a side stream (warms up the allocator and the library before capture)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for t in range(2):
            step_fn(t)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()


def capture(step_fn, n_graph, first=0):
    """Captures steps first .. first + n_graph - 1 as one graph (after two eager warm-up steps)."""
    side_warmup(step_fn)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t in range(first, first + n_graph):
            step_fn(t)
    torch.cuda.synchronize()
    return g


class Replayer:
    """Graphs of n_graph consecutive steps, replayed in order.  Steps alternate between two
    buffers by the parity of their index, so for an odd n_graph two graphs (steps 0 .. n-1 and
    n .. 2n-1) alternate and the chain stays serial: step t + 1 always reads step t's output."""

    def __init__(self, step_fn, n_graph):
        self.n = n_graph
        self.graphs = [capture(step_fn, n_graph)]
        if n_graph % 2:
            self.graphs.append(capture(step_fn, n_graph, first=n_graph))
        self.done = 0   # replays so far

    def replay(self):
        self.graphs[self.done % len(self.graphs)].replay()
        self.done += 1

    def next_first_step(self):
        """Index (mod 2 significant) of the first step of the next replay."""
        return self.done * self.n


def time_graph(step_fn, n_graph, warmup, steps, rep=None):
    """Replays graphs of n_graph consecutive steps for about `warmup` steps untimed, then
    steps/n_graph times timed, HIP events between replays on the replay stream.  Returns
    (total seconds, per-replay seconds list, the Replayer)."""
    rep = rep if rep is not None else Replayer(step_fn, n_graph)
    for _ in range(max(1, warmup // n_graph)):
        rep.replay()
    torch.cuda.synchronize()
    reps = steps // n_graph
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for r in range(reps):
        rep.replay()
        ev[r + 1].record()
    torch.cuda.synchronize()
    per = [ev[r].elapsed_time(ev[r + 1]) / 1e3 for r in range(reps)]
    return ev[0].elapsed_time(ev[reps]) / 1e3, per, rep


def cpu_info():
    """(CPU model name, threads this process may use) of the host the bench runs on."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    n = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return model, n


def baseline(v1, s1, vn, sn, n, unit):
    """cpu_baseline object: the oracle on all usable cores (value, cores) with the one-core run
    beside it, and the host's CPU model."""
    model, _ = cpu_info()
    return dict(value=vn, unit=unit, cores=n, kind="oracle", sample=sn, cpu_model=model,
                one_core=dict(value=v1, unit=unit, cores=1, sample=s1))


def cpu_baseline_stack(cpu_layers, wl, n_tokens):
    """The oracle (fp64 truth mode) through the first layers of the stack: one thread on n_tokens
    chained tokens, and all usable cores on independent sequences (one token each per layer call,
    outputs rounded to bf16 between layers as in the stack)."""
    import oracle
    ors = [oracle.Layer(c["w_router"], c["t_gate"], c["t_up"], c["t_down"], c["s_gate"],
                        c["s_up"], c["s_down"], pre_rmsnorm=wl.pre_rmsnorm, top_k=wl.top_k)
           for c in cpu_layers]
    scale = wl.n_layers / len(ors)
    x = synth.activations(wl, n_tokens, seed=4242)
    t0 = time.perf_counter()
    for t in range(n_tokens):
        oracle.decode_stack(ors, x[t].double().numpy(), 1)
    dt1 = time.perf_counter() - t0
    _, n = cpu_info()
    T = 4 * n
    xs = synth.activations(wl, T, seed=4243).double().numpy()
    t0 = time.perf_counter()
    cur = xs
    for layer in ors:
        out, _, _, _ = oracle.moe_layer(layer, cur, n_threads=n)
        cur = oracle.round_bf16(out)
    dtn = time.perf_counter() - t0
    return baseline(
        n_tokens / (dt1 * scale),
        "%d chained tokens through %d of the %d layers, one thread, %.1f s; rate scaled to %d layers"
        % (n_tokens, len(ors), wl.n_layers, dt1, wl.n_layers),
        T / (dtn * scale),
        "%d independent sequences, one step through %d of the %d layers, %d threads, %.1f s; rate "
        "scaled to %d layers" % (T, len(ors), wl.n_layers, n, dtn, wl.n_layers),
        n, "tok/s")


def run_stack(args):
    wl = synth.STACK24_B1
    n_cpu_layers = 0 if args.no_cpu_baseline else 3
    layers, cpu_layers = [], []
    for l in range(wl.n_layers):
        layer, cpu = build_layer(wl, l, keep_cpu=l < n_cpu_layers)
        layers.append(layer)
        if cpu is not None:
            cpu_layers.append(cpu)
    torch.cuda.synchronize()
    assert all(int(l.bad_count.item()) == 0 for l in layers)
    x0 = synth.activations(wl, 1, device="cuda")[0]
    bufs = [x0.clone(), torch.empty_like(x0)]
    ws = torch.empty(tw.decode_workspace_bytes(layers), dtype=torch.uint8, device="cuda")

    def step(t):
        tw.ternary_moe_ffn_decode(layers, bufs[t % 2], out=bufs[(t + 1) % 2], workspace=ws)

    # graphs of G = min(--steps, 256) consecutive steps, replayed at least 20 times in the timed
    # region (every replay is a sample); the steps actually timed are reported
    G = min(args.steps, args.graph_steps)
    reps = max(20, -(-args.steps // G))
    steps = reps * G
    total, per, rep = time_graph(step, G, args.warmup, steps)
    # the health word after the timed replays: a hand-off wait that ran out would have ended a
    # launch early (and made it look fast)
    health = tw.decode_error_flag(layers, ws)
    if health != 0:
        log("stack24_b1: decode health word %#x after the timed replays" % health)
        sys.exit(3)
    # one more replay against the same G steps run eagerly from the same state, bit for bit
    first = rep.next_first_step()
    src, dst = bufs[first % 2], bufs[(first + G) % 2]
    start = src.clone()
    rep.replay()
    torch.cuda.synchronize()
    replayed = dst.clone()
    health = tw.decode_error_flag(layers, ws)
    src.copy_(start)
    for t in range(first, first + G):
        step(t)
    torch.cuda.synchronize()
    if health != 0 or tw.decode_error_flag(layers, ws) != 0 or \
            not torch.equal(replayed.view(torch.int16), dst.view(torch.int16)):
        log("stack24_b1: graph replay differs from the eager chain of the same %d steps" % G)
        sys.exit(3)
    requested = args.steps
    args.steps = steps
    ms_per_step = total / args.steps * 1e3
    bytes_per_step = accounting.stack_bytes_per_token(wl)
    tok_s = args.steps / total
    achieved = bytes_per_step / (total / args.steps) / 1e9
    per_tok_us = sorted(p / G * 1e6 for p in per)
    log("stack24_b1: %.2f us/token median over %d replays of %d steps (min %.2f, p90 %.2f)" % (
        per_tok_us[len(per_tok_us) // 2], len(per), G, per_tok_us[0],
        per_tok_us[int(0.9 * (len(per_tok_us) - 1))]))
    cpu = cpu_baseline_stack(cpu_layers, wl, args.cpu_tokens) if cpu_layers else None
    traffic = traffic_from_profiles("stack24_b1")
    return dict(
        metric=METRIC, value=tok_s, unit="tok/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=ms_per_step, higher_is_better=True, scaling="weak",
        vs_baseline=None,
        dtype="int8 digit planes x ternary -> exact int32 sums (activations kept to 14 bits below "
              "their max |x|), fp32 scales/SiLU/gates/combine, bf16 I/O",
        data="synthetic",
        config=dict(workload="stack24_b1", layers=wl.n_layers, d_model=wl.d_model,
                    n_experts=wl.n_experts, d_ff=wl.d_ff, top_k=wl.top_k, batch=1,
                    graph_steps=G, replays=len(per), requested_steps=requested,
                    bytes_per_token=bytes_per_step,
                    us_per_token_median=per_tok_us[len(per_tok_us) // 2],
                    us_per_token_min=per_tok_us[0],
                    us_per_token_p90=per_tok_us[int(0.9 * (len(per_tok_us) - 1))],
                    health_word=0, replay_equals_eager=True),
        roofline=dict(bound="hbm", achieved=achieved, peak=accounting.HBM_PEAK_BPS / 1e9,
                      unit="GB/s", frac=achieved * 1e9 / accounting.HBM_PEAK_BPS,
                      traffic=traffic,
                      kernel="k_persist<2048,512,8>: one launch per step runs all 24 layers "
                             "(timed with the small word-clearing kernel launched before it)",
                      bytes_per_launch=bytes_per_step,
                      us_per_launch=total / args.steps * 1e6),
        cpu_baseline=cpu,
    )


def run_single_layer(args, name):
    wl = synth.WORKLOADS[name]
    n_copies = 8
    T = wl.batch
    act = wl.act
    layers, cpu0 = [], None
    for c in range(n_copies):
        layer, cpu = build_layer(wl, c, keep_cpu=(c == 0 and not args.no_cpu_baseline))
        layers.append(layer)
        cpu0 = cpu0 if cpu is None else cpu
    xs = [synth.activations(wl, T, device="cuda", stream=c) for c in range(n_copies)]
    outs = [torch.empty((T, wl.d_model), dtype=torch.bfloat16 if wl.out_dtype == "bf16"
                        else torch.float32, device="cuda") for _ in range(n_copies)]
    # distinct experts per copy, from the routing the call itself will compute; the int8
    # prefill-shaped workload takes its routing as an input (computed here, outside the timing)
    distinct, routing = [], []
    for c in range(n_copies):
        _, ids, gates = tw.moe_route_topk(xs[c], layers[c].w_router, wl.top_k)
        distinct.append(int(torch.unique(ids).numel()))
        routing.append((ids, gates) if name == "prefill_4096" else (None, None))
    if T == 1:
        ws = torch.empty(tw.decode_workspace_bytes([layers[0]]), dtype=torch.uint8, device="cuda")

        def step(t):
            c = t % n_copies
            tw.ternary_moe_ffn_decode([layers[c]], xs[c][0], out=outs[c][0], workspace=ws)
    else:
        ws = torch.empty(tw.batched_workspace_bytes(layers[0], T, act), dtype=torch.uint8,
                         device="cuda")

        def step(t):
            c = t % n_copies
            tw.ternary_moe_ffn_batched(layers[c], xs[c], act=act, out=outs[c], workspace=ws,
                                       expert_ids=routing[c][0], gate_w=routing[c][1])

    G = args.graph_steps
    steps = max(1, round(args.steps / G)) * G   # whole replays; every replay rotates all copies
    total, per, _ = time_graph(step, G, args.warmup, steps)
    args.steps = steps
    bytes_per_step = sum(accounting.layer_bytes(wl, T, distinct[t % n_copies])
                         for t in range(G)) / G
    achieved = bytes_per_step / (total / args.steps) / 1e9
    if name == "prefill_4096":
        ops = accounting.int8_ops(wl, T * wl.top_k)
        tops = ops / (total / args.steps) / 1e12
        roof = dict(bound="mfma", achieved=tops, peak=accounting.INT8_MFMA_PEAK_OPS / 1e12,
                    unit="TOP/s", frac=tops * 1e12 / accounting.INT8_MFMA_PEAK_OPS,
                    traffic=traffic_from_profiles(name),   # HBM bytes per k_pf_expert dispatch
                    kernel="one call: quantise x, group, k_pf_expert<2048,512>, combine",
                    ops_per_call=ops, hbm_gb_s=achieved)
    else:
        roof = dict(bound="hbm", achieved=achieved, peak=accounting.HBM_PEAK_BPS / 1e9,
                    unit="GB/s", frac=achieved * 1e9 / accounting.HBM_PEAK_BPS,
                    traffic=traffic_from_profiles(name), kernel="one call")
    return dict(
        metric="%s tokens/s (one layer, %d tokens per call)" % (name, T), value=T * args.steps / total,
        unit="tok/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=total / args.steps * 1e3, higher_is_better=True, scaling="weak",
        vs_baseline=None, dtype="int8xint8->int32, fp32", data="synthetic",
        config=dict(workload=name, batch=T, act=act, layer_copies=n_copies,
                    distinct_experts=distinct, bytes_per_step=bytes_per_step),
        roofline=roof,
        cpu_baseline=cpu_baseline_layer(cpu0, wl, name) if cpu0 is not None else None,
    )


def cpu_baseline_layer(cpu, wl, name):
    """The oracle on a bounded sample of one single-layer workload: truth mode (fp64) for the
    float paths, the int8 spec mode (routing from the oracle's own router) for int8 activations;
    one thread on a few tokens, and all usable cores on more."""
    import oracle
    lay = oracle.Layer(cpu["w_router"], cpu["t_gate"], cpu["t_up"], cpu["t_down"], cpu["s_gate"],
                       cpu["s_up"], cpu["s_down"], pre_rmsnorm=wl.pre_rmsnorm, top_k=wl.top_k)
    _, n = cpu_info()
    int8 = wl.act == "int8"
    n1 = 8 if wl.batch > 1 else 4
    nn = min(wl.batch, 32 * n) if int8 else max(wl.batch, 8 * n)

    def run(T, threads):
        x = synth.activations(wl, T, seed=4244).double().numpy()
        t0 = time.perf_counter()
        if int8:
            ids, g, _ = oracle.route(lay, x, n_threads=threads)
            oracle.ffn_batch_i8(lay, x.astype("float32"), ids, g.astype("float32"), n_threads=threads)
        else:
            oracle.moe_layer(lay, x, n_threads=threads)
        return time.perf_counter() - t0

    d1, dn = run(n1, 1), run(nn, n)
    mode = "int8 spec mode, oracle routing" if int8 else "fp64 truth mode"
    return baseline(n1 / d1, "%d tokens of %s (%s), one thread, %.1f s" % (n1, name, mode, d1),
                    nn / dn, "%d tokens of %s (%s), %d threads, %.1f s" % (nn, name, mode, n, dn),
                    n, "tok/s")


def run_quantize(args):
    """ternary_quantize of one full layer's float expert weights (gate, up, down: 805 M bf16
    weights, 1.6 GB, larger than the last-level cache) per step."""
    wl = synth.QUANTIZE_LAYER
    w = synth.float_expert_weights(wl, 0, device="cuda")
    mats = [w["w_gate"], w["w_up"], w["w_down"]]
    outs = [(torch.empty(m.shape[:-1] + (m.shape[-1] // 4,), dtype=torch.uint8, device="cuda"),
             torch.empty(m.shape[:-1], dtype=torch.float32, device="cuda")) for m in mats]
    torch.cuda.synchronize()

    def step(t):
        for m, (p, sc) in zip(mats, outs):
            tw.ternary_quantize(m, packed=p, scales=sc)

    G = min(args.graph_steps, 16)
    steps = max(G, (args.steps // 10) // G * G)
    total, _, _ = time_graph(step, G, min(args.warmup, 4 * G), steps)
    sec = total / steps
    n_w = sum(m.numel() for m in mats)
    bytes_per_step = accounting.quantize_bytes(wl)
    achieved = bytes_per_step / sec / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        import oracle  # the CPU baseline leg: the oracle as it stands, one thread
        sample = mats[0].reshape(-1, wl.d_model)[:131072].cpu()
        t0 = time.perf_counter()
        oracle.quantize_absmean(sample)
        dt = time.perf_counter() - t0
        cpu = dict(value=sample.numel() / dt, unit="weights/s", cores=1, kind="oracle",
                   sample="131072 rows of 2048 bf16 weights (the gate matrix, %.1f s), one thread" % dt)
    return dict(
        metric="quantize_layer weights/s (float -> packed ternary, one layer's experts)",
        value=n_w / sec, unit="weights/s", n_gpus=1, steps=steps, warmup=args.warmup,
        ms_per_step=sec * 1e3, higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype="bf16 -> 2-bit codes + fp32 scales", data="synthetic",
        config=dict(workload="quantize_layer", weights=n_w, bytes_per_step=bytes_per_step),
        roofline=dict(bound="hbm", achieved=achieved, peak=accounting.HBM_PEAK_BPS / 1e9,
                      unit="GB/s", frac=achieved * 1e9 / accounting.HBM_PEAK_BPS, traffic=None,
                      kernel="k_quant_absmean<bf16> x 3 (gate, up, down)"),
        cpu_baseline=cpu,
    )


def run_gemv(args, layout):
    """ternary_gemv_i8 over the gate and up rows of one layer's 256 experts (262144 rows of 2048
    weights), packed two bits per weight (layout 2) or five weights per byte (layout 3).  Four
    weight copies are rotated, so that the codes come from HBM rather than the last-level cache."""
    rows, cols = synth.GEMV_ROWS, synth.GEMV_COLS
    n_copies = 4
    mats = []
    for c in range(n_copies):
        w = synth.trits((rows, cols), "cuda", 1100 + c, 0, "gate")
        codes = tw.ternary_pack3(w) if layout == 3 else tw.ternary_pack(w)
        del w
        sc = synth.uniform((rows,), 0.01, 0.1, "cuda", 1100 + c, 0, "s_gate").contiguous()
        mats.append((codes, sc))
    xq = synth.int8_codes(cols, "cuda", 1100)
    xs = torch.tensor([0.01], dtype=torch.float32, device="cuda")
    ys = [torch.empty(rows, dtype=torch.float32, device="cuda") for _ in range(n_copies)]
    torch.cuda.synchronize()

    def step(t):
        c = t % n_copies
        tw.ternary_gemv_i8(mats[c][0], layout, mats[c][1], cols, xq, xs, out=ys[c])

    G = min(args.graph_steps, 64)
    steps = max(G, (args.steps // 4) // G * G)
    total, _, _ = time_graph(step, G, min(args.warmup, 4 * G), steps)
    sec = total / steps
    bytes_per_step = accounting.gemv_bytes(rows, cols, layout)
    achieved = bytes_per_step / sec / 1e9
    name = "gemv_base3" if layout == 3 else "gemv_2bit"
    return dict(
        metric="%s weights/s (int8 ternary GEMV, %d rows x %d weights)" % (name, rows, cols),
        value=rows * cols / sec, unit="weights/s", n_gpus=1, steps=steps, warmup=args.warmup,
        ms_per_step=sec * 1e3, higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype="int8 x ternary -> int32, fp32 out", data="synthetic",
        config=dict(workload=name, rows=rows, cols=cols, layout=layout,
                    row_bytes=tw.ternary_pack3_row_bytes(cols) if layout == 3 else cols // 4,
                    weight_copies=n_copies, bytes_per_step=bytes_per_step),
        roofline=dict(bound="hbm", achieved=achieved, peak=accounting.HBM_PEAK_BPS / 1e9,
                      unit="GB/s", frac=achieved * 1e9 / accounting.HBM_PEAK_BPS, traffic=None,
                      kernel="k_gemv_i8<%d>" % layout),
        cpu_baseline=None,
    )


def run_attention(args, one=False):
    """Decode attention of one token through the 24 layers' caches: 6 global layers over the pages'
    640-token context and 18 windowed layers over their 512-slot rings (16 query heads over 4 KV
    heads of 128, bf16).  12 step copies of all 24 caches (320 MB) are rotated, so that the caches
    come from HBM rather than the 256 MB last-level cache.  one: attention_decode_one (one launch
    per layer) instead of attention_decode (two)."""
    H, Hkv, dh = synth.ATTN_HEADS, synth.ATTN_KV_HEADS, synth.ATTN_HEAD_DIM
    n_layers = synth.ATTN_GLOBAL_LAYERS + synth.ATTN_WINDOW_LAYERS
    slots = [synth.ATTN_CONTEXT if (l % 4) == 3 else synth.ATTN_WINDOW for l in range(n_layers)]
    n_copies = 12
    caches = []
    for c in range(n_copies):
        caches.append([synth.attention_inputs(slots[l], "cuda", seed=2000 + c, layer=l)
                       for l in range(n_layers)])
    outs = [torch.empty((H, dh), dtype=torch.float32, device="cuda") for _ in range(n_layers)]
    if one:
        ws = tw.attention_decode_one_workspace(H, dh, max(slots))
    else:
        ws = torch.empty(tw.attention_decode_workspace_bytes(H, dh, max(slots)), dtype=torch.uint8,
                         device="cuda")
    torch.cuda.synchronize()

    def step(t):
        c = t % n_copies
        for l in range(n_layers):
            q, k, v = caches[c][l]
            if one:
                tw.attention_decode_one(q, k, v, ws, out=outs[l])
            else:
                tw.attention_decode(q, k, v, out=outs[l], workspace=ws)

    G = min(args.graph_steps, 48)
    steps = max(G, (args.steps // 8) // G * G)
    total, _, _ = time_graph(step, G, min(args.warmup, 4 * G), steps)
    sec = total / steps
    bytes_per_step = sum(2 * n * Hkv * dh * 2 + 2 * H * dh + 4 * H * dh for n in slots)
    achieved = bytes_per_step / sec / 1e9
    return dict(
        metric="attention_24l steps/s (decode attention of one token through 24 layers' caches)",
        value=1.0 / sec, unit="tok/s", n_gpus=1, steps=steps, warmup=args.warmup,
        ms_per_step=sec * 1e3, higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype="bf16 in, fp32 sums and out", data="synthetic",
        config=dict(workload="attention_24l_one" if one else "attention_24l", heads=H, kv_heads=Hkv, head_dim=dh,
                    global_layers=synth.ATTN_GLOBAL_LAYERS, global_slots=synth.ATTN_CONTEXT,
                    window_layers=synth.ATTN_WINDOW_LAYERS, window_slots=synth.ATTN_WINDOW,
                    step_copies=n_copies, bytes_per_step=bytes_per_step),
        roofline=dict(bound="hbm", achieved=achieved, peak=accounting.HBM_PEAK_BPS / 1e9,
                      unit="GB/s", frac=achieved * 1e9 / accounting.HBM_PEAK_BPS, traffic=None,
                      kernel=("k_attn_one<4>" if one else "k_attn_part<4> + k_attn_merge") + ", 24 layer calls per step"),
        cpu_baseline=None,
    )


def run_flash_head(args):
    """Approximate output head: 151,936 tokens in 4,748 clusters of 32, hidden size 2048, the top
    512 clusters (67 MB of head rows per call).  Eight hidden states rotate, so that consecutive
    calls select different clusters and their rows (together most of the 622 MB head) come from
    HBM rather than the 256 MB last-level cache."""
    ncl, cs, d, top = synth.HEAD_CLUSTERS, synth.HEAD_CLUSTER_SIZE, synth.HEAD_D, synth.HEAD_TOP
    f = synth.head_inputs(ncl, cs, d, "cuda", seed=3000)
    hs = [synth.head_hidden(d, "cuda", seed=3000, stream=i) for i in range(8)]
    ws = torch.empty(tw.lib().flash_head_workspace_bytes(ncl), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()

    def step(t):
        tw.flash_head(hs[t % 8], f["centroids"], f["centroid_scales"], f["w_clustered"],
                      f["member_ids"], top, workspace=ws)

    G = min(args.graph_steps, 64)
    steps = max(G, (args.steps // 4) // G * G)
    total, _, _ = time_graph(step, G, min(args.warmup, 4 * G), steps)
    sec = total / steps
    bytes_per_step = (ncl * d // 2 + 4 * ncl + 2 * d + top * cs * d * 2 + top * cs * 4
                      + top * cs * 8 + 4 * top)
    achieved = bytes_per_step / sec / 1e9
    return dict(
        metric="flash_head calls/s (4,748 clusters of 32 tokens, top 512, hidden 2048)",
        value=1.0 / sec, unit="calls/s", n_gpus=1, steps=steps, warmup=args.warmup,
        ms_per_step=sec * 1e3, higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype="int4 x int8 -> int32 scores, bf16 x bf16 -> fp32 logits", data="synthetic",
        config=dict(workload="flash_head", clusters=ncl, cluster_size=cs, hidden=d, top=top,
                    hidden_states=8, bytes_per_step=bytes_per_step),
        roofline=dict(bound="hbm", achieved=achieved, peak=accounting.HBM_PEAK_BPS / 1e9,
                      unit="GB/s", frac=achieved * 1e9 / accounting.HBM_PEAK_BPS, traffic=None,
                      kernel="k_head_score<1> + k_head_rank + k_head_logits<4>"),
        cpu_baseline=None,
    )


PHASE_NAMES = ["x gather + router (to the router barrier)", "logit gather (wave 0)", "top-k (wave 0)",
               "top-k to its barrier", "gate/up loads + dots (to the h-publish barrier)",
               "h publish + h gather (wave 0)", "down + max + digit planes (to the combine barrier)",
               "combine + publish (to the end of the layer)"]


def run_phases(args):
    """Per-layer phase breakdown of the stacked decode from the measurement build
    (libternary_moe_phases.so, -DTW_PHASE_TIMES): thread 0 of every workgroup stores the 100 MHz
    wall clock at each phase boundary of every layer; means over workgroups, layers 1..23 and
    20 steps.  The stores add a little time to every layer, so the total is above the product
    build's."""
    import numpy as np
    wl = synth.STACK24_B1
    layers = [build_layer(wl, l)[0] for l in range(wl.n_layers)]
    x = synth.activations(wl, 1, device="cuda")[0]
    ws = torch.zeros(tw.decode_workspace_bytes(layers), dtype=torch.uint8, device="cuda")
    off = tw.lib().ternary_moe_decode_error_offset((tw.TwLayer * len(layers))(*[l.c for l in layers]),
                                                   len(layers)) + 256
    nwg, nl, ns = 256, 32, 10
    bufs = [x.clone(), torch.empty_like(x)]
    runs = []
    for it in range(40):
        tw.ternary_moe_ffn_decode(layers, bufs[it % 2], out=bufs[(it + 1) % 2], workspace=ws)
        if it >= 20:
            torch.cuda.synchronize()
            assert tw.decode_error_flag(layers, ws) == 0
            raw = ws[off:off + nwg * nl * ns * 8].cpu().view(torch.int64).numpy()
            runs.append(raw.reshape(nwg, nl, ns)[:, :wl.n_layers, :].astype(np.float64) / 100.0)
    ts = np.stack(runs)                       # [run, workgroup, layer, stamp] in us
    L = slice(1, wl.n_layers)
    order = [0, 1, 7, 8, 2, 3, 4, 5, 6]       # the stamps in time order within a layer
    d = np.diff(ts[..., order], axis=3)[:, :, L, :]
    phases = {n: round(float(d[..., i].mean()), 3) for i, n in enumerate(PHASE_NAMES)}
    period = float((ts[:, :, 2:wl.n_layers, 0] - ts[:, :, 1:wl.n_layers - 1, 0]).mean())
    skew = {str(p): round(float((ts[:, :, L, p].max(axis=1) - ts[:, :, L, p].min(axis=1)).mean()), 3)
            for p in order}
    lastpub = ts[:, :, 0:wl.n_layers - 1, 6].max(axis=1)
    handoffs = {
        "last residual published -> first / last router done":
            [round(float((ts[:, :, 1:, 1].min(axis=1) - lastpub).mean()), 3),
             round(float((ts[:, :, 1:, 1].max(axis=1) - lastpub).mean()), 3)],
        "last logit published -> first / last top-k done":
            [round(float((ts[:, :, L, 2].min(axis=1) - ts[:, :, L, 1].max(axis=1)).mean()), 3),
             round(float((ts[:, :, L, 2].max(axis=1) - ts[:, :, L, 1].max(axis=1)).mean()), 3)],
        "last h published -> first / last h gathered":
            [round(float((ts[:, :, L, 4].min(axis=1) - ts[:, :, L, 3].max(axis=1)).mean()), 3),
             round(float((ts[:, :, L, 4].max(axis=1) - ts[:, :, L, 3].max(axis=1)).mean()), 3)],
    }
    for n, v in phases.items():
        log("  %-52s %.3f us" % (n, v))
    log("  layer period %.3f us" % period)
    return dict(metric="stack24_b1 per-layer phase breakdown (measurement build)", value=period,
                unit="us per layer", n_gpus=1, steps=20, warmup=20, ms_per_step=None,
                higher_is_better=False, scaling="weak", vs_baseline=None, dtype="as stack24_b1",
                data="synthetic",
                config=dict(workload="stack24_phases", layers=wl.n_layers, layers_averaged="1..23",
                            workgroups=nwg, phases_us=phases, stamp_skew_us=skew,
                            handoffs_us=handoffs),
                roofline=None, cpu_baseline=None)


def run_copy_calib(args):
    """A plain device-to-device copy of a known size (4 x 1 GiB), for scaling the FETCH_SIZE and
    WRITE_SIZE hardware counters of the measured kernels."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    reps = 4
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    return dict(metric="device copy GB/s (read + write)", value=2 * n * reps / dt / 1e9, unit="GB/s",
                n_gpus=1, steps=reps, warmup=0, ms_per_step=dt / reps * 1e3,
                higher_is_better=True, scaling="weak", vs_baseline=None, dtype="u8",
                data="synthetic", config=dict(workload="copy_calib", bytes_per_copy=n),
                roofline=None, cpu_baseline=None)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2560)
    ap.add_argument("--warmup", type=int, default=512)
    ap.add_argument("--graph-steps", type=int, default=256)
    ap.add_argument("--workload", default="stack24_b1",
                    choices=["stack24_b1", "stack24_phases", "layer_b1", "batched_b64", "batched_b64_int8",
                             "prefill_4096", "quantize_layer", "gemv_2bit", "gemv_base3",
                             "attention_24l", "attention_24l_one", "flash_head", "copy_calib"])
    ap.add_argument("--cpu-tokens", type=int, default=16)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.workload == "stack24_phases":
        from ternary_weight_moe_amd import build as twb
        tw.LIB_PATH = twb.PHASES_LIB   # the measurement build, before the library is loaded
    tw.lib()
    if args.workload == "stack24_b1":
        res = run_stack(args)
    elif args.workload == "stack24_phases":
        res = run_phases(args)
    elif args.workload == "copy_calib":
        res = run_copy_calib(args)
    elif args.workload == "quantize_layer":
        res = run_quantize(args)
    elif args.workload == "attention_24l":
        res = run_attention(args)
    elif args.workload == "attention_24l_one":
        res = run_attention(args, one=True)
    elif args.workload == "flash_head":
        res = run_flash_head(args)
    elif args.workload in ("gemv_2bit", "gemv_base3"):
        res = run_gemv(args, 3 if args.workload == "gemv_base3" else 2)
    else:
        res = run_single_layer(args, args.workload)
    res["device"] = torch.cuda.get_device_properties(0).gcnArchName
    res["rocm"] = torch.version.hip
    print(json.dumps(res))


if __name__ == "__main__":
    main()
