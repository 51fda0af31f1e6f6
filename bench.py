#!/usr/bin/env python3
"""Throughput of the gated delta-rule step on one MI355X (gfx950).

Default workload (the headline one): batched decode, B=64 independent sequences
of one token each, Hk=16, Hv=32, dk=dv=128, tiled k-head map, bf16 activations
drawn N(0,1), fp32 state N(0, 0.02^2), conv width 4 with carried state. One step
is one pass of the whole decode path in one launch: gdn_decode_layer (depthwise
conv + SiLU with the conv window carried between two buffers, split, L2 norm of
q/k, gates, recurrence, gated RMS norm). The same inputs are reused every step;
the state evolves.

Metric: decode state GB/s = 2 * B * Hv * dv * dk * 4 bytes (the fp32 state read
and written once) / step time, the definition of the ferrox-core gdn.rs
throughput probe. Also reported on the same JSON line:
  * roofline: the layer kernel's algorithmic bytes per launch / its average
    duration (one HIP event pair around K back-to-back launches, timed right
    after the K steps), against the 8 TB/s HBM peak; traffic from the committed
    rocprofv3 FETCH/WRITE counter summary when it was taken on the current
    kernel source, else null;
  * two_launch: the same step as gdn_conv_update then gdn_decode_step;
  * rotating: the step cycling through 4 independent state sets (537 MB,
    larger than the 256 MB Infinity Cache), so the state cannot stay cached;
    timed with the GDN_STREAM_STATE cache hint and without it, over 1000 steps
    whatever --steps says; pct_hbm_peak_cache_free and roofline_cache_free come
    from it (the headline's 128 MiB state partly stays in that cache);
  * verify: multi-token verify decode (T = 2, 4, 8 tokens per call) at B=64;
  * deep_model: 48 layers per token at Hv=48, B=1 and B=32, uncaptured and as
    one HIP graph; B=32 (4.8 GB of state) with GDN_STREAM_STATE;
  * prefill: chunked prefill tokens/s at B=1, T=4096; prefill_varlen: 8 packed
    sequences of 512..8192 tokens;
  * cpu_baseline: the CPU oracle on the host cores (all the GPU's share, and one
    thread): the decode step, the T=4096 and varlen prefill calls, the 48-layer
    model per layer (extrapolated per token); the CPU model and nproc.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
VARLEN_LENGTHS = (512, 1024, 2048, 3072, 4096, 5120, 6144, 8192)
ROTATING_STEPS = 1000
METRIC = "decode state GB/s (% HBM peak); prefill tokens/s at Hv=32,d=128"


def kernel_source_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "gated_deltanet_linear_step_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(summary_name, source_hash, key="hbm_bytes_per_dispatch"):
    """Bytes per dispatch from a committed counter summary, if it matches the source."""
    path = os.path.join(ROOT, "profiles", summary_name)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    t = re.search(key + r":\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != source_hash:
        return None
    return float(t.group(1))


def decode_bench(args, torch, ops, synth, rot_steps=ROTATING_STEPS):
    """The headline: B=64 decode steps, each one gdn_decode_layer launch (conv +
    L2 norm + gates + recurrence + gated norm), with the conv state alternating
    between two buffers; then the same step as gdn_conv_update + gdn_decode_step
    (two launches) for comparison, a burst of back-to-back layer launches (the
    roofline) and a rotating 4-state-set variant beyond the Infinity Cache."""
    dev = torch.device("cuda:0")
    B, Hk, Hv, d = 64, 16, 32, 128
    QK = Hk * d
    QKV = 2 * QK + Hv * d
    sets = []
    nsets = 4
    for i in range(nsets):
        W = synth.decode_batch(seed=2 + 1000 * i, B=B, Hk=Hk, Hv=Hv, dk=d, dv=d,
                               head_map=synth.TILED)
        S = {k: (v.to(dev).contiguous() if hasattr(v, "to") else v) for k, v in W.items()}
        S["conv_b"] = torch.empty_like(S["conv_state"])
        S["y"] = torch.empty((B, QKV), dtype=torch.float32, device=dev)
        S["out"] = torch.empty((B, Hv, d), dtype=torch.bfloat16, device=dev)
        kw = dict(Hk=Hk, Hv=Hv, dk=d, dv=d, head_map=synth.TILED, batch=B, a=S["a"], b=S["b"],
                  decay_param=S["A_log"], dt_bias=S["dt_bias"], z=S["z"], norm_weight=S["norm_w"])
        x = S["x"]
        # layer[j]: conv state read from buffer j, written to the other one;
        # layer_stream: the same calls with GDN_STREAM_STATE (for the rotating sets,
        # whose 537 MB of state does not stay in the 256 MB Infinity Cache)
        pairs = ((S["conv_state"], S["conv_b"]), (S["conv_b"], S["conv_state"]))
        S["layer"] = [ops.prepare_decode_layer(x[:, :QK], x[:, QK:2 * QK], x[:, 2 * QK:],
                                               S["state"], S["conv_w"], cin, cout, S["out"], **kw)
                      for cin, cout in pairs]
        S["layer_stream"] = [ops.prepare_decode_layer(x[:, :QK], x[:, QK:2 * QK], x[:, 2 * QK:],
                                                      S["state"], S["conv_w"], cin, cout,
                                                      S["out"], stream_state=True, **kw)
                             for cin, cout in pairs]
        S["parity"] = 0
        S["conv"] = ops.prepare_conv_update(S["x"], S["conv_w"], S["conv_state"], S["y"])
        y = S["y"]
        S["dec"] = ops.prepare_decode_step(y[:, :QK], y[:, QK:2 * QK], y[:, 2 * QK:], S["state"],
                                           S["out"], **kw)
        sets.append(S)
    main = sets[0]

    def step(S, key="layer"):
        S[key][S["parity"]].launch()
        S["parity"] ^= 1

    def timed(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n, time.perf_counter() - w0

    for _ in range(args.warmup):
        step(main)
    K = args.steps
    # timed region 1 (the metric): K whole steps, one event pair around them
    ms_step, wall = timed(lambda i: step(main), K)
    # timed region 2 (the roofline): K more layer launches back to back on the same
    # stream -> the layer kernel's average duration
    dec_ms, _ = timed(lambda i: step(main), K)
    # the same step in two launches (conv update, then the decode step)
    if main["parity"]:  # the two-launch path keeps the window in conv_state
        main["conv_state"].copy_(main["conv_b"])
        main["parity"] = 0

    def two(i):
        main["conv"].launch()
        main["dec"].launch()
    for _ in range(args.warmup):
        two(0)
    ms_two, _ = timed(two, K)

    state_bytes = 2 * B * Hv * d * d * 4
    # layer kernel algorithmic bytes: state r+w; bf16 x read (q/k/v before the
    # conv), conv window read and written, conv taps; z, a, b in; bf16 out;
    # per-head parameters
    act_bytes = B * QKV * 2 + 2 * B * QKV * 3 * 2 + QKV * 4 * 2 + B * Hv * d * 2 \
        + 2 * B * Hv * 2 + B * Hv * d * 2 + Hv * 4 * 2 + d * 4
    dec_bytes = state_bytes + act_bytes
    value = state_bytes / (ms_step * 1e-3) / 1e9

    # rotating variant: 4 state sets, > Infinity Cache; with GDN_STREAM_STATE (the
    # caller's hint for exactly this case), then without it. Its length does not
    # follow --steps: ROTATING_STEPS steps (about 50 ms) always.
    for _ in range(nsets * 4):
        for S in sets:
            step(S, "layer_stream")
    Kr = rot_steps
    ms_rot, _ = timed(lambda i: step(sets[i % nsets], "layer_stream"), Kr)
    for _ in range(nsets * 4):
        for S in sets:
            step(S)
    ms_rot_plain, _ = timed(lambda i: step(sets[i % nsets]), Kr)

    src_hash = kernel_source_hash(["gdn_decode.hip", "gdn_device.h", "gdn_kernels.h"])
    traffic = read_traffic("decode_layer_b64_bf16_traffic.md", src_hash)
    achieved = dec_bytes / (dec_ms * 1e-3) / 1e9
    rot_achieved = dec_bytes / (ms_rot * 1e-3) / 1e9
    res = dict(
        value=value, ms_per_step=ms_step, wall_s=wall,
        state_residency="cache-resident: the 128 MiB state of this workload stays partly in "
                        "the 256 MB Infinity Cache between steps; the rotating leg and "
                        "roofline_cache_free give the rate with the state streamed from HBM",
        roofline=dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=achieved / HBM_PEAK_GBS, traffic=traffic,
                      traffic_note="L2-to-fabric bytes (FETCH_SIZE + WRITE_SIZE, calibrated on a "
                                   "copy); the counters do not tell Infinity-Cache hits from "
                                   "HBM reads",
                      kernel="gdn decode_kernel<dk=128,dv=128,waves=8,bf16,conv K=4> "
                             "(gdn_decode_layer)", bytes_per_launch=dec_bytes,
                      avg_launch_us=dec_ms * 1e3, kernel_source_sha256_16=src_hash,
                      state="cache-resident (128 MiB, fits the 256 MB Infinity Cache)"),
        roofline_cache_free=dict(bound="hbm", achieved=rot_achieved, peak=HBM_PEAK_GBS,
                                 unit="GB/s", frac=rot_achieved / HBM_PEAK_GBS,
                                 kernel="gdn decode_kernel<dk=128,dv=128,waves=16,bf16,conv K=4,"
                                        "non-temporal> (gdn_decode_layer, GDN_STREAM_STATE)",
                                 traffic=read_traffic("decode_layer_b64_bf16_traffic.md", src_hash,
                                                      "stream_bytes_per_dispatch"),
                                 bytes_per_launch=dec_bytes, avg_launch_us=ms_rot * 1e3,
                                 steps=Kr, state="streamed: 4 state sets, 537 MB, cycled"),
        two_launch=dict(step="gdn_conv_update + gdn_decode_step", ms_per_step=ms_two,
                        value=state_bytes / (ms_two * 1e-3) / 1e9, unit="GB/s"),
        rotating=dict(sets=nsets, footprint_mb=nsets * (state_bytes // 2) / 1e6, steps=Kr,
                      stream_state=True, ms_per_step=ms_rot,
                      pct_hbm_peak=100 * state_bytes / (ms_rot * 1e-3) / 1e9 / HBM_PEAK_GBS,
                      value=state_bytes / (ms_rot * 1e-3) / 1e9, unit="GB/s",
                      ms_per_step_no_hint=ms_rot_plain,
                      value_no_hint=state_bytes / (ms_rot_plain * 1e-3) / 1e9),
        config=dict(workload="batched decode: B=64 x 1 token, Hk=16, Hv=32, dk=dv=128, tiled map, "
                             "bf16 N(0,1) activations, fp32 state N(0,0.02^2), conv K=4",
                    batch=B, tokens_per_seq=1, Hk=Hk, Hv=Hv, dk=d, dv=d, head_map="tiled",
                    act_dtype="bf16", state_dtype="f32", out_dtype="bf16",
                    step="gdn_decode_layer (conv + norm + gates + recurrence + gated norm, "
                         "one launch)"),
    )
    return res


def verify_bench(torch, ops, synth, Ts=(2, 4, 8), calls=200, warmup=20):
    """Multi-token verify decode at B=64 (the headline shapes): one gdn_decode_layer
    call carries T tokens per sequence through the state, which is read and written
    once per call."""
    dev = torch.device("cuda:0")
    B, Hk, Hv, d = 64, 16, 32, 128
    QK = Hk * d
    res = {}
    for T in Ts:
        W = synth.decode_batch(seed=20 + T, B=B, Hk=Hk, Hv=Hv, dk=d, dv=d, T=T,
                               head_map=synth.TILED)
        S = {k: (v.to(dev).contiguous() if hasattr(v, "to") else v) for k, v in W.items()}
        cb = torch.empty_like(S["conv_state"])
        out = torch.empty((B * T, Hv, d), dtype=torch.bfloat16, device=dev)
        x = S["x"]
        calls_ = [ops.prepare_decode_layer(
            x[:, :QK], x[:, QK:2 * QK], x[:, 2 * QK:], S["state"], S["conv_w"], ci, co, out,
            Hk=Hk, Hv=Hv, dk=d, dv=d, head_map=synth.TILED, batch=B, tokens_per_seq=T, a=S["a"],
            b=S["b"], decay_param=S["A_log"], dt_bias=S["dt_bias"], z=S["z"],
            norm_weight=S["norm_w"]) for ci, co in ((S["conv_state"], cb), (cb, S["conv_state"]))]
        for i in range(warmup):
            calls_[i & 1].launch()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(calls):
            calls_[i & 1].launch()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / calls
        state_bytes = 2 * B * Hv * d * d * 4
        res[f"T{T}"] = dict(ms_per_call=ms, tokens_per_s=B * T / (ms * 1e-3),
                            state_GBps=state_bytes / (ms * 1e-3) / 1e9,
                            state_GBps_per_token=state_bytes * T / (ms * 1e-3) / 1e9)
    return dict(workload="multi-token verify decode: B=64 x T tokens per call, Hk=16, Hv=32, "
                         "dk=dv=128, tiled map, bf16 N(0,1), one gdn_decode_layer call",
                **res)


HEAD_SHAPES = ((32, 32), (64, 64), (96, 96), (128, 128), (64, 128), (128, 64), (128, 256),
               (256, 128), (256, 256))


def head_shapes_bench(torch, ops, synth, calls=300, warmup=30):
    """The fused decode layer at every built (dk, dv) head shape: B=64 x 1 token,
    Hk=16, Hv=32, tiled map, bf16 N(0,1) activations, fp32 state; state GB/s over
    back-to-back launches (the state is read and written once per launch), without
    and with the GDN_STREAM_STATE hint (the hint is meant for states that do not
    stay in the 256 MB Infinity Cache: here 128x256, 256x128 and 256x256)."""
    dev = torch.device("cuda:0")
    B, Hk, Hv = 64, 16, 32
    res = {}
    for dk, dv in HEAD_SHAPES:
        W = synth.decode_batch(seed=30 + dk + dv, B=B, Hk=Hk, Hv=Hv, dk=dk, dv=dv,
                               head_map=synth.TILED)
        S = {k: (v.to(dev).contiguous() if hasattr(v, "to") else v) for k, v in W.items()}
        cb = torch.empty_like(S["conv_state"])
        out = torch.empty((B, Hv, dv), dtype=torch.bfloat16, device=dev)
        x, QK = S["x"], Hk * dk
        state_bytes = 2 * B * Hv * dv * dk * 4
        r = {}
        for hint in (False, True):
            calls_ = [ops.prepare_decode_layer(
                x[:, :QK], x[:, QK:2 * QK], x[:, 2 * QK:], S["state"], S["conv_w"], ci, co, out,
                Hk=Hk, Hv=Hv, dk=dk, dv=dv, head_map=synth.TILED, batch=B, a=S["a"], b=S["b"],
                decay_param=S["A_log"], dt_bias=S["dt_bias"], z=S["z"], norm_weight=S["norm_w"],
                stream_state=hint)
                for ci, co in ((S["conv_state"], cb), (cb, S["conv_state"]))]
            for i in range(warmup):
                calls_[i & 1].launch()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for i in range(calls):
                calls_[i & 1].launch()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / calls
            gbps = state_bytes / (ms * 1e-3) / 1e9
            sfx = "_hint" if hint else ""
            r.update({f"us_per_launch{sfx}": ms * 1e3, f"state_GBps{sfx}": gbps,
                      f"pct_hbm_peak{sfx}": 100 * gbps / HBM_PEAK_GBS})
            del calls_
        res[f"{dk}x{dv}"] = r
        del S, W
    return dict(workload="fused decode layer per head shape (dk x dv): B=64 x 1 token, Hk=16, "
                         "Hv=32, tiled map, bf16 N(0,1), fp32 state, back-to-back launches; "
                         "*_hint: with GDN_STREAM_STATE",
                **res)


def deep_model_bench(torch, ops, synth, batches=(1, 32), layers=48, steps=(100, 20)):
    """Deep-model decode: Hk=16, Hv=48, d=128, `layers` layers applied in sequence per
    token, each with its own seeded taps, gates, norm, state and conv window (seed
    4*1000 + layer); one token step = `layers` gdn_decode_layer launches. Timed
    uncaptured and as one captured HIP graph (two token steps per graph, so the conv
    windows alternate back to their first buffers). When the stack's states exceed the
    256 MB Infinity Cache (B=32: 4.8 GB; B=1: 151 MB does not), the calls carry
    GDN_STREAM_STATE, as a caller of such a stack would set it."""
    dev = torch.device("cuda:0")
    Hk, Hv, d = 16, 48, 128
    QK = Hk * d
    res = {}
    for B, nsteps in zip(batches, steps):
        stream_state = layers * B * Hv * d * d * 4 > 256 * 2**20
        cap = torch.cuda.Stream()
        Ls = []
        for layer in range(layers):
            W = synth.decode_batch(seed=4 * 1000 + layer, B=B, Hk=Hk, Hv=Hv, dk=d, dv=d,
                                   head_map=synth.TILED)
            S = {k: (v.to(dev).contiguous() if hasattr(v, "to") else v) for k, v in W.items()}
            S["cb"] = torch.empty_like(S["conv_state"])
            S["out"] = torch.empty((B, Hv, d), dtype=torch.bfloat16, device=dev)
            x = S["x"]
            kw = dict(Hk=Hk, Hv=Hv, dk=d, dv=d, head_map=synth.TILED, batch=B, a=S["a"],
                      b=S["b"], decay_param=S["A_log"], dt_bias=S["dt_bias"], z=S["z"],
                      norm_weight=S["norm_w"], stream_state=stream_state)
            pairs = ((S["conv_state"], S["cb"]), (S["cb"], S["conv_state"]))
            S["eager"] = [ops.prepare_decode_layer(x[:, :QK], x[:, QK:2 * QK], x[:, 2 * QK:],
                                                   S["state"], S["conv_w"], ci, co, S["out"],
                                                   **kw) for ci, co in pairs]
            S["cap"] = [ops.prepare_decode_layer(x[:, :QK], x[:, QK:2 * QK], x[:, 2 * QK:],
                                                 S["state"], S["conv_w"], ci, co, S["out"],
                                                 stream=cap, **kw) for ci, co in pairs]
            Ls.append(S)

        def token(par, key):
            for S in Ls:
                S[key][par].launch()

        for i in range(4):
            token(i & 1, "eager")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(nsteps):
            token(i & 1, "eager")
        e1.record()
        torch.cuda.synchronize()
        ms_eager = e0.elapsed_time(e1) / nsteps
        if nsteps % 2:
            token(1, "eager")  # back to parity 0
        graph = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=cap):
            token(0, "cap")
            token(1, "cap")
        torch.cuda.synchronize()
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = max(1, nsteps // 2)
        g0.record()
        for _ in range(reps):
            graph.replay()
        g1.record()
        torch.cuda.synchronize()
        ms_graph = g0.elapsed_time(g1) / (2 * reps)
        state_bytes = 2 * layers * B * Hv * d * d * 4
        res[f"B{B}"] = dict(ms_per_token_step=ms_eager, ms_per_token_step_graph=ms_graph,
                            state_GBps=state_bytes / (ms_eager * 1e-3) / 1e9,
                            state_GBps_graph=state_bytes / (ms_graph * 1e-3) / 1e9,
                            state_bytes_per_step=state_bytes, stream_state=stream_state)
        del graph, Ls
        torch.cuda.empty_cache()
    return dict(workload=f"deep-model decode: {layers} layers x gdn_decode_layer per token, "
                         "Hk=16, Hv=48, dk=dv=128, tiled map, bf16 N(0,1), fp32 states",
                **res)


PREFILL_OTHER_SHAPES = ((32, 32), (64, 64), (96, 96), (64, 128), (128, 64), (128, 256),
                        (256, 128), (256, 256))


def prefill_shapes_bench(torch, ops, synth, calls=10, warmup=2):
    """The chunked prefill at the other built head shapes (the f32 path: preparation
    kernel per (chunk, k-head), carry per (sequence, v-head, 32 dv rows)):
    one sequence of T=4096 and the 8-sequence varlen batch, Hk=16, Hv=32, bf16
    N(0,1) inputs, raw gates, core output; tokens/s, and the state-and-activation
    bytes per call over the call time against 8 TB/s."""
    res = {}
    for dk, dv in PREFILL_OTHER_SHAPES:
        r = {}
        for name, lengths, hm, std in (("T4096", (4096,), synth.GROUPED, 0.0),
                                       ("varlen", VARLEN_LENGTHS, synth.TILED, 0.02)):
            pre = prefill_bench(torch, ops, synth, lengths=lengths, head_map=hm, state_std=std,
                                seed=3, calls=calls, warmup=warmup, dk=dk, dv=dv)
            r[name] = dict(us_per_call=pre["ms_per_call"] * 1e3, tokens_per_s=pre["tokens_per_s"],
                           hbm_frac=pre["roofline"]["frac"])
        res[f"{dk}x{dv}"] = r
    return dict(workload="chunked prefill per head shape (dk x dv), Hk=16, Hv=32, bf16 N(0,1), "
                         "raw gates, f32 core output: one T=4096 sequence and the 8-sequence "
                         "varlen batch (30,208 tokens)", **res)


def prefill_bench(torch, ops, synth, *, lengths=(4096,), head_map=None, state_std=0.0,
                  out_dtype=None, seed=3, calls=20, warmup=5, workload=None, dk=128, dv=128):
    """Chunked prefill over packed sequences of the given lengths, Hk=16, Hv=32,
    d=128, bf16 N(0,1) inputs, raw gates with A_log ~ U[-2,0], q/k L2-normalised
    in-op, initial states N(0, state_std^2), core output (no gated norm). Defaults:
    config 3 (one sequence of 4096 tokens, grouped map, zero state, f32 out)."""
    dev = torch.device("cuda:0")
    Hk, Hv = 16, 32
    head_map = synth.GROUPED if head_map is None else head_map
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    P = synth.prefill(seed=seed, lengths=list(lengths), Hk=Hk, Hv=Hv, dk=dk, dv=dv,
                      head_map=head_map, state_std=state_std)
    T = int(P["cu_seqlens"][-1])
    N = len(lengths)
    g = lambda t: t.reshape(T, -1).to(dev).contiguous()  # noqa: E731
    q, k, v, a, b = g(P["q"]), g(P["k"]), g(P["v"]), g(P["a"]), g(P["b"])
    state0 = P["state"].to(dev).contiguous()
    state = state0.clone()
    out = torch.empty((T, Hv, dv), dtype=out_dtype, device=dev)
    cu_h = P["cu_seqlens"].contiguous()
    cu_d = cu_h.to(dev)
    need = ops.prefill_workspace_bytes(Hk=Hk, Hv=Hv, dk=dk, dv=dv, num_seqs=N, total_tokens=T)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    call = ops.prepare_prefill_chunked(q, k, v, state, cu_d, cu_h, out, ws, Hk=Hk, Hv=Hv, dk=dk,
                                       dv=dv, head_map=head_map, a=a, b=b,
                                       decay_param=P["A_log"].to(dev),
                                       dt_bias=P["dt_bias"].to(dev))
    for _ in range(warmup):
        state.copy_(state0)
        call.launch()
    times = []
    for _ in range(calls):
        state.copy_(state0)  # every call starts from the same state (outside the timed span)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        call.launch()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    times.sort()
    ms = times[len(times) // 2]
    C = 64
    chunks = sum((n + C - 1) // C for n in lengths)
    # algorithmic MFMA work of the chunked form, per (chunk, v-head): U, W (2 C^2 d
    # each), W S^T, Q S^T, D^T K (2 C d^2 each), Aqk D (2 C^2 d); per (chunk, k-head):
    # K K^T and Q K^T (2 C^2 d each)
    flops = chunks * (Hv * (2 * C * C * dv + 2 * C * C * dk + 2 * C * C * dv + 3 * 2 * C * dk * dv)
                      + Hk * 2 * 2 * C * C * dk)
    # HBM bytes: bf16 q, k, v, a, b in; the output; the states read and written once
    osz = 4 if out_dtype == torch.float32 else 2
    hbm = T * (2 * Hk * dk + Hv * dv + 2 * Hv) * 2 + T * Hv * dv * osz + 2 * N * Hv * dk * dv * 4
    t = ms * 1e-3
    traffic = None
    if tuple(lengths) == (4096,) and (dk, dv) == (128, 128):
        traffic = read_traffic("prefill_t4096_traffic.md",
                               kernel_source_hash(["gdn_prefill.hip", "gdn_device.h", "gdn_kernels.h"]))
    return dict(workload=workload, tokens=T, sequences=N, chunks=chunks,
                tokens_per_s=T / t, ms_per_call=ms, calls=calls, unit="tokens/s",
                mfma_flops=flops, mfma_util=flops / t / (MFMA_F16_PEAK_TFLOPS * 1e12),
                roofline=dict(bound="hbm", achieved=hbm / t / 1e9, peak=HBM_PEAK_GBS,
                              unit="GB/s", frac=hbm / t / 1e9 / HBM_PEAK_GBS, bytes=hbm,
                              traffic=traffic, traffic_note="L2-to-fabric bytes per call (prep + "
                              "carry), from the committed counter summary when it matches the "
                              "sources; the excess over `bytes` is the workspace's round trip"))


def counter_pass(torch, ops, synth, steps=10, copy_mib=256):
    """For HBM-byte counters: `steps` steps of each decode leg of the headline
    workload (fused layer, two-launch step), 4 calls of the T=4096 prefill, then
    `steps` copies of copy_mib MiB
    (read and written once each: 2 * copy_mib MiB of traffic per dispatch), whose
    counter readings calibrate the decode kernels'."""
    args = argparse.Namespace(warmup=2, steps=steps)
    decode_bench(args, torch, ops, synth, rot_steps=4 * steps)
    prefill_bench(torch, ops, synth, calls=3, warmup=1)
    n = copy_mib * 2 ** 20 // 4
    src = torch.randn(n, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"[bench] counter pass: {steps} decode steps, {steps} copies of {copy_mib} MiB",
          file=sys.stderr, flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(seconds):
    """The f64 CPU oracle as it stands, on the host cores, as a baseline only (never
    the target): the B=64 decode step (the headline's unit, state GB/s) on all the
    threads the host grants this GPU and on one thread; the T=4096 and the varlen
    prefill calls whole; the 48-layer model per layer, extrapolated per token. The
    oracle's drivers spread independent sequences (decode) or (sequence, v-head)
    pairs (prefill) over threads; each unit is the sequential f64 recurrence."""
    import numpy as np
    import oracle
    from gated_deltanet_linear_step_amd import synth

    f = lambda t: t.double().numpy()  # noqa: E731
    nproc = os.cpu_count() or 1
    threads = max(1, min(16, nproc))  # a one-GPU host's share of the cores: 16
    res = dict(kind="oracle", cores=threads, nproc=nproc, cpu_model=cpu_model())

    # --- the headline decode step: B=64, one token, conv + core, state GB/s
    B, Hk, Hv, d = 64, 16, 32, 128
    W = synth.decode_batch(seed=2, B=B, Hk=Hk, Hv=Hv, dk=d, dv=d, head_map=synth.TILED)
    state_bytes = 2 * B * Hv * d * d * 4

    def decode_rate(nthreads, budget):
        S, cs = f(W["state"]), f(W["conv_state"])
        steps, t0 = 0, time.perf_counter()
        while True:
            _, cs, S = oracle.batch(B=B, T=1, Hk=Hk, Hv=Hv, dk=d, dv=d, head_map=oracle.MAP_TILED,
                                    S0=S, a=f(W["a"]), b=f(W["b"]), decay_param=f(W["A_log"]),
                                    dt_bias=f(W["dt_bias"]), z=f(W["z"]), norm_w=f(W["norm_w"]),
                                    x=f(W["x"]), conv_w=f(W["conv_w"]), conv_state=cs,
                                    nthreads=nthreads)
            steps += 1
            if time.perf_counter() - t0 >= budget:
                return steps, (time.perf_counter() - t0) / steps

    steps, dt = decode_rate(threads, 0.35 * seconds)
    res.update(value=state_bytes / dt / 1e9, unit="GB/s", ms_per_step=dt * 1e3,
               sample=f"{steps} decode steps of the B=64 workload (conv + core, f64 oracle, "
                      f"{threads} threads over sequences); GB/s counts fp32 state bytes")
    steps1, dt1 = decode_rate(1, 0.2 * seconds)
    res["single_thread"] = dict(value=state_bytes / dt1 / 1e9, unit="GB/s", cores=1,
                                ms_per_step=dt1 * 1e3, sample=f"{steps1} decode steps, one thread")

    # --- the chunked-prefill workloads through the token-by-token oracle
    def prefill_rate(P, nthreads, heads=None, seqs=None):
        cu = [int(c) for c in P["cu_seqlens"]]
        if seqs is not None:  # a prefix of the packed sequences
            cu = cu[:seqs + 1]
        T = cu[-1]
        g = lambda t: f(t[:T])  # noqa: E731
        t0 = time.perf_counter()
        oracle.packed(g(P["q"]), g(P["k"]), g(P["v"]), f(P["state"][:len(cu) - 1]), P["head_map"],
                      cu, a=g(P["a"]), b=g(P["b"]), decay_param=f(P["A_log"]),
                      dt_bias=f(P["dt_bias"]), nthreads=nthreads, heads=heads)
        dt = time.perf_counter() - t0
        nh = Hv if heads is None else len(heads)
        return T, dt, T * nh / Hv / dt  # tokens/s of a whole (all-heads) call

    P3 = synth.prefill(seed=3, lengths=[4096], head_map=synth.GROUPED)
    T3, dt3, rate3 = prefill_rate(P3, threads)
    _, dt31, rate31 = prefill_rate(P3, 1, heads=[0, 1])
    res["prefill_t4096"] = dict(value=rate3, unit="tokens/s", cores=threads, s_per_call=dt3,
                                sample="one whole T=4096 call, all 32 v-heads",
                                single_thread=dict(value=rate31, unit="tokens/s", cores=1,
                                                   sample="2 of 32 v-heads of the T=4096 call on "
                                                          "one thread, scaled to 32 (extrapolated)"))
    P5 = synth.prefill(seed=5, lengths=list(VARLEN_LENGTHS), head_map=synth.TILED, state_std=0.02)
    T5, dt5, rate5 = prefill_rate(P5, threads)
    res["prefill_varlen"] = dict(value=rate5, unit="tokens/s", cores=threads, s_per_call=dt5,
                                 sample=f"one whole varlen call: 8 sequences, {T5} tokens, "
                                        "all 32 v-heads")

    # --- the 48-layer model, per layer, extrapolated per token
    deep = {}
    for Bd in (1, 32):
        Ld = synth.decode_batch(seed=4000, B=Bd, Hk=16, Hv=48, dk=d, dv=d, head_map=synth.TILED)
        S, cs = f(Ld["state"]), f(Ld["conv_state"])
        n, t0 = 0, time.perf_counter()
        while n < 1 or time.perf_counter() - t0 < 0.05 * seconds:
            _, cs, S = oracle.batch(B=Bd, T=1, Hk=16, Hv=48, dk=d, dv=d, head_map=oracle.MAP_TILED,
                                    S0=S, a=f(Ld["a"]), b=f(Ld["b"]), decay_param=f(Ld["A_log"]),
                                    dt_bias=f(Ld["dt_bias"]), z=f(Ld["z"]), norm_w=f(Ld["norm_w"]),
                                    x=f(Ld["x"]), conv_w=f(Ld["conv_w"]), conv_state=cs,
                                    nthreads=threads)
            n += 1
        per_layer = (time.perf_counter() - t0) / n
        sb = 2 * 48 * Bd * 48 * d * d * 4
        deep[f"B{Bd}"] = dict(ms_per_layer=per_layer * 1e3, ms_per_token_step=48 * per_layer * 1e3,
                              state_GBps=sb / (48 * per_layer) / 1e9, layers_timed=n,
                              sample=f"{n} layer steps timed, extrapolated to 48 layers per "
                                     "token (extrapolated)")
    res["deep_model"] = dict(cores=threads, **deep)
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="time budget of the CPU baseline's decode and deep-model legs; the "
                         "prefill legs are whole calls")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-verify", action="store_true",
                    help="skip the multi-token, 48-layer and head-shape decode legs")
    ap.add_argument("--counter-pass", action="store_true",
                    help="short run for rocprofv3 --pmc: a few decode steps, then a plain "
                         "256 MiB device copy of known size (the counters' calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this library has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)

    import torch
    from gated_deltanet_linear_step_amd import ops, synth
    ops.load()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)

    if args.counter_pass:
        counter_pass(torch, ops, synth)
        return
    print(f"[bench] decode B=64: warmup {args.warmup}, steps {args.steps}", file=sys.stderr,
          flush=True)
    dec = decode_bench(args, torch, ops, synth)
    print(f"[bench] decode {dec['value']:.1f} GB/s, {dec['ms_per_step'] * 1e3:.2f} us/step",
          file=sys.stderr, flush=True)
    line = dict(metric=METRIC, value=round(dec["value"], 2), unit="GB/s", n_gpus=1,
                steps=args.steps, warmup=args.warmup, ms_per_step=dec["ms_per_step"],
                higher_is_better=True, scaling="weak", vs_baseline=None, dtype="f32",
                data="synthetic", config=dec["config"],
                pct_hbm_peak=round(100 * dec["value"] / HBM_PEAK_GBS, 2),
                pct_hbm_peak_cache_free=round(dec["rotating"]["pct_hbm_peak"], 2),
                state_residency=dec["state_residency"],
                roofline=dec["roofline"], roofline_cache_free=dec["roofline_cache_free"],
                two_launch=dec["two_launch"], rotating=dec["rotating"])
    if not args.no_verify:
        print("[bench] multi-token verify decode, T=2,4,8", file=sys.stderr, flush=True)
        line["verify"] = verify_bench(torch, ops, synth)
        print("[bench] deep-model decode, 48 layers, B=1 and B=32", file=sys.stderr, flush=True)
        line["deep_model"] = deep_model_bench(torch, ops, synth)
        print("[bench] decode layer per head shape", file=sys.stderr, flush=True)
        line["head_shapes"] = head_shapes_bench(torch, ops, synth)
    if not args.no_prefill:
        print("[bench] prefill T=4096", file=sys.stderr, flush=True)
        pre = prefill_bench(
            torch, ops, synth,
            workload="chunked prefill: B=1, T=4096, C=64, Hk=16, Hv=32, dk=dv=128, grouped map, "
                     "bf16 N(0,1) inputs, q/k L2-normalised, raw gates, zero initial state, "
                     "f32 core output")
        print(f"[bench] prefill {pre['tokens_per_s'] / 1e6:.2f} M tokens/s, "
              f"{pre['ms_per_call'] * 1e3:.1f} us/call", file=sys.stderr, flush=True)
        line["prefill"] = pre
        print("[bench] varlen prefill, 8 sequences", file=sys.stderr, flush=True)
        var = prefill_bench(
            torch, ops, synth, lengths=VARLEN_LENGTHS, head_map=synth.TILED, state_std=0.02,
            out_dtype=torch.bfloat16, seed=5,
            workload="varlen chunked prefill: 8 sequences of 512..8192 tokens (30,208 packed), "
                     "C=64, Hk=16, Hv=32, dk=dv=128, tiled map, bf16 N(0,1) inputs, raw gates, "
                     "initial states N(0,0.02^2), bf16 core output")
        print(f"[bench] varlen prefill {var['tokens_per_s'] / 1e6:.2f} M tokens/s, "
              f"{var['ms_per_call'] * 1e3:.1f} us/call", file=sys.stderr, flush=True)
        line["prefill_varlen"] = var
        print("[bench] prefill per head shape", file=sys.stderr, flush=True)
        line["prefill_head_shapes"] = prefill_shapes_bench(torch, ops, synth)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
