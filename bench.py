#!/usr/bin/env python3
"""Throughput of the JetBlock hot path (libjetblock) on one MI355X.

One step = one JetBlock-2B-shape prefill of a 65,536-token sequence (B=1,
H=12, dk=96, dv=256, d_model=1536, chunk 64) followed by 128 decode steps
for 256 sequences of the same shape from seeded fp32 states.  Inputs are
seeded synthetic tensors already resident in HBM.  value = tokens processed
per second over the whole step (65,536 prefill + 32,768 decode tokens).

Each decode step is one jb_decode_step call, a single kernel launch
(generator, conv and state update fused).  HIP events on the launching
stream bracket every jb_prefill call and every 16th decode launch
(--event-every; recording events costs the stream a few microseconds, so a
pair around every launch would slow the timed loop), which gives the
per-kernel averages the roofline figures use.

Prints one JSON line on stdout; progress goes to stderr.
  python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload 2b|4b]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = 2500.0    # MI355X dense fp16/bf16 matrix peak, TFLOP/s


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def prefill_flops_per_token(s) -> float:
    """Algorithmic flops per token of the chunked prefill (C = 64):
    H (6 C dk + 4 C dv + 6 dk dv) + 2 D G + 2 G 4H + 8 H dv."""
    C, G = 64, 32
    return (s.H * (6 * C * s.dk + 4 * C * s.dv + 6 * s.dk * s.dv) + 2 * s.d_model * G + 2 * G * 4 * s.H
            + 8 * s.H * s.dv)


def prefill_bytes_per_token(s, out_bytes: int) -> float:
    """Compulsory HBM bytes per token: x, q, k, v (bf16), alpha, beta (f32), o."""
    return 2 * s.d_model + 2 * 2 * s.H * s.dk + 2 * s.H * s.dv + 8 * s.H + out_bytes * s.H * s.dv


def decode_step_bytes(s, out_bytes: int) -> float:
    """Compulsory HBM bytes of one jb_decode_step launch for B sequences: per (sequence, head)
    the fp32 state read and written once, q, k, v_t (bf16), the 3-row cache read and written,
    alpha, beta (f32) and o; per sequence x_t (bf16); once, the generator weights W1, W2."""
    per_unit = 2 * s.dk * s.dv * 4 + 2 * s.dk * 2 + s.dv * 2 + 2 * 3 * s.dv * 2 + 8 + s.dv * out_bytes
    return s.B * s.H * per_unit + s.B * s.d_model * 2 + (32 * s.d_model + 4 * s.H * 32) * 2


def decode_static_bytes(s, out_bytes: int) -> float:
    """Compulsory HBM bytes of one jb_decode_step_static launch: per (sequence, head) the fp32
    state read and written once, q, k, v_t (bf16), the three 3-row caches read and written,
    alpha, beta (f32) and o; once, the conv weights (f32, 4 per channel)."""
    per_unit = (2 * s.dk * s.dv * 4 + 2 * s.dk * 2 + s.dv * 2 + 2 * 3 * (2 * s.dk + s.dv) * 2 + 8
                + s.dv * out_bytes)
    return s.B * s.H * per_unit + s.H * (2 * s.dk + s.dv) * 16


def measured_traffic(profile: str, sources: list[str]):
    """HBM bytes per launch of a kernel, from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by a plain-copy calibration), or None when the
    summary is missing or the kernel's sources changed since the counters were taken."""
    import hashlib
    try:
        text = open(os.path.join(ROOT, "profiles", profile)).read()
        h = hashlib.sha256(b"".join(open(os.path.join(ROOT, f), "rb").read() for f in sources)).hexdigest()[:16]
    except OSError:
        return None
    fields = dict(line.split(": ", 1) for line in text.splitlines() if ": " in line and line[:1].isalpha())
    if fields.get("source_sha256_16", "").strip() != h:
        return None
    return float(fields["traffic_bytes_per_launch"])


def projection_flops_per_token(s) -> float:
    """Matrix flops per token of the input projections: 2 D (2 H dk + H dv + 32 + 2 H)."""
    return 2.0 * s.d_model * (2 * s.H * s.dk + s.H * s.dv + 32 + 2 * s.H)


def measure_from_x(jb, inputs, torch, sp, out_dt, reps: int = 5, dec_reps: int = 30):
    """The block from its layer input x (outside the timed step): jb_project alone and
    jb_prefill_from_x at the prefill shape (`reps` calls each), jb_decode_step_from_x at the
    decode shape (`dec_reps` calls), each after 3 warm-up calls and bracketed by HIP events on
    the launching stream."""
    dev = torch.device("cuda:0")
    p = inputs.projection_inputs(sp, seed=2, device=dev)
    stream = torch.cuda.current_stream()
    pshape = jb.make_shape(sp.B, sp.T, sp.H, sp.dk, sp.dv, sp.d_model, jb.JB_BF16,
                           jb.JB_BF16 if out_dt == torch.bfloat16 else jb.JB_F32)
    ws_p = jb.workspace(jb.project_workspace_size(pshape), dev)
    ws_x = jb.workspace(jb.prefill_from_x_workspace_size(pshape), dev)
    o = torch.empty((sp.B, sp.T, sp.H, sp.dv), dtype=out_dt, device=dev)
    S = torch.empty((sp.B, sp.H, sp.dk, sp.dv), dtype=torch.float32, device=dev)

    def timed(fn, n=reps):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    ms_proj = timed(lambda: jb.project(**p, ws=ws_p, stream=stream))
    # one decode step from x_t at the decode shape (projections over the batch + the step)
    sd = inputs.B2_DECODE if sp.H == inputs.B2_DECODE.H else inputs.B4_DECODE
    pd = inputs.projection_inputs(sd, seed=3, device=dev)
    Wd = {k: pd[k] for k in ("Wq", "Wk", "Wv", "Wa", "Wb", "W1", "W2", "ba", "bb")}
    st = inputs.state_inputs(sd, seed=3, device=dev)
    xt = pd["x"][:, 0].contiguous()
    od = torch.empty((sd.B, sd.H, sd.dv), dtype=out_dt, device=dev)
    dshape = jb.make_shape(sd.B, 1, sd.H, sd.dk, sd.dv, sd.d_model)
    ws_d = jb.workspace(jb.decode_step_from_x_workspace_size(dshape), dev)
    us_dec = 1e3 * timed(lambda: jb.decode_step_from_x(st["S"], st["cache"], xt, **Wd, out_dtype=out_dt, o=od,
                                                       ws=ws_d, stream=stream), dec_reps)
    ms_x = timed(lambda: jb.prefill_from_x(**p, out_dtype=out_dt, o=o, S_final=S, want_conv_out=False, ws=ws_x,
                                           stream=stream))
    tok = sp.B * sp.T
    proj_tf = projection_flops_per_token(sp) * tok / (ms_proj * 1e-3) / 1e12
    return dict(call="jb_prefill_from_x (projections from x, generator, recurrence)", tokens=tok,
                ms=round(ms_x, 4), tokens_per_s=round(tok / (ms_x * 1e-3), 1),
                decode_step_from_x=dict(call="jb_decode_step_from_x", B=sd.B, us=round(us_dec, 2),
                                        tokens_per_s=round(sd.B / (us_dec * 1e-6), 1)),
                project=dict(call="jb_project (q, k, v, gates, taps from x)", ms=round(ms_proj, 4), bound="mfma",
                             achieved=round(proj_tf, 2), peak=MFMA_PEAK_TFLOPS, unit="TFLOP/s",
                             frac=round(proj_tf / MFMA_PEAK_TFLOPS, 4),
                             flops_per_call=projection_flops_per_token(sp) * tok))


def measure_static(jb, inputs, torch, sp, sd, p, d, out_dt, reps: int = 3):
    """The static-conv block, the one JetBlock replaces, on the same inputs (outside the timed
    step): jb_prefill_static at the prefill shape and jb_decode_step_static at the decode shape,
    each averaged over `reps` calls bracketed by HIP events on the launching stream."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    w = inputs.static_conv_inputs(sp, seed=5, device=dev)
    o = torch.empty((sp.B, sp.T, sp.H, sp.dv), dtype=out_dt, device=dev)
    S = torch.empty((sp.B, sp.H, sp.dk, sp.dv), dtype=torch.float32, device=dev)
    pshape = jb.make_shape(sp.B, sp.T, sp.H, sp.dk, sp.dv, sp.d_model, jb.JB_BF16,
                           jb.JB_BF16 if out_dt == torch.bfloat16 else jb.JB_F32)
    need = jb.prefill_static_workspace_size(pshape)
    ws = jb.workspace(need, dev) if need else None

    def timed(fn, n=reps):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    ms_pre = timed(lambda: jb.prefill_static(p["q"], p["k"], p["v"], p["alpha"], p["beta"], w["wq"], w["wk"], w["wv"],
                                             out_dtype=out_dt, o=o, S_final=S, want_cache_out=False, ws=ws,
                                             stream=stream))
    wd = inputs.static_conv_inputs(sd, seed=6, device=dev)
    Sd = d["S"].clone()
    od = torch.empty((sd.B, sd.H, sd.dv), dtype=out_dt, device=dev)
    us_dec = 1e3 * timed(lambda: jb.decode_step_static(Sd, wd["cache_q"], wd["cache_k"], wd["cache_v"], d["q"][0],
                                                       d["k"][0], d["v"][0], d["alpha"][0], d["beta"][0], wd["wq"],
                                                       wd["wk"], wd["wv"], out_dtype=out_dt, o=od, stream=stream))
    out_bytes = 2 if out_dt == torch.bfloat16 else 4
    dec_gbs = decode_static_bytes(sd, out_bytes) / (us_dec * 1e-6) / 1e9
    tok = sp.B * sp.T
    return dict(prefill=dict(call="jb_prefill_static", ms=round(ms_pre, 4), tokens_per_s=round(tok / (ms_pre * 1e-3), 1)),
                decode=dict(call="jb_decode_step_static (decode_seq_static_kernel)", B=sd.B, us=round(us_dec, 2),
                            tokens_per_s=round(sd.B / (us_dec * 1e-6), 1), hbm_GBs=round(dec_gbs, 1),
                            hbm_frac=round(dec_gbs / HBM_PEAK_GBS, 4),
                            bytes_per_launch=decode_static_bytes(sd, out_bytes)))


def measure_serving(jb, inputs, torch, sp, sd, out_dt, n_req: int, lo: int, hi: int, steps: int = 16, reps: int = 2):
    """A serving batch (outside the timed step): n_req requests of lo..hi tokens at the
    prefill shape's heads, prefilled as one packed batch (jb_prefill_varlen), then `steps`
    decode steps of the whole batch from the prefill's states and caches (jb_decode_step).
    Each part averaged over HIP events on the launching stream."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    lengths = inputs.request_lengths(n_req, lo, hi, seed=1)
    total = sum(lengths)
    p = inputs.packed_prefill_inputs(lengths, sp.H, sp.dk, sp.dv, sp.d_model, seed=4, device=dev)
    cu = p["cu_seqlens"]
    o = torch.empty((total, sp.H, sp.dv), dtype=out_dt, device=dev)
    S = torch.empty((n_req, sp.H, sp.dk, sp.dv), dtype=torch.float32, device=dev)
    cache = torch.empty((n_req, 3, sp.H, sp.dv), dtype=torch.bfloat16, device=dev)
    shape = jb.make_shape(n_req, max(lengths), sp.H, sp.dk, sp.dv, sp.d_model)
    ws = jb.workspace(jb.prefill_varlen_workspace_size(shape, total), dev)

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    ms_pre = timed(lambda: jb.prefill_varlen(cu, p["x"], p["q"], p["k"], p["v"], p["alpha"], p["beta"], p["W1"],
                                             p["W2"], max_seqlen=max(lengths), out_dtype=out_dt, o=o, S_final=S,
                                             conv_out=cache, ws=ws, stream=stream), reps)
    del p, o
    d = inputs.decode_inputs(inputs.Shape(B=n_req, T=1, H=sd.H, dk=sd.dk, dv=sd.dv, d_model=sd.d_model),
                             steps=steps, seed=8, device=dev, with_state=False)
    od = torch.empty((n_req, sd.H, sd.dv), dtype=out_dt, device=dev)
    state = dict(t=0)

    def step():
        t = state["t"] % steps
        state["t"] += 1
        jb.decode_step(S, cache, d["x"][t], d["q"][t], d["k"][t], d["v"][t], d["alpha"][t], d["beta"][t], d["W1"],
                       d["W2"], out_dtype=out_dt, o=od, stream=stream)

    us_dec = 1e3 * timed(step, steps)
    flops = prefill_flops_per_token(sp) * total
    tf = flops / (ms_pre * 1e-3) / 1e12
    return dict(requests=n_req, lengths=f"uniform {lo}..{hi} (seeded)", tokens=total,
                prefill=dict(call="jb_prefill_varlen", ms=round(ms_pre, 3), tokens_per_s=round(total / (ms_pre * 1e-3), 1),
                             mfma_frac=round(tf / MFMA_PEAK_TFLOPS, 4)),
                decode=dict(call="jb_decode_step (states handed over from the prefill)", B=n_req,
                            us=round(us_dec, 2), tokens_per_s=round(n_req / (us_dec * 1e-6), 1)))


def measure_training(jb, inputs, torch, sp, B: int, T: int, reps: int = 3):
    """Training at the prefill shape's heads (outside the timed step): B sequences of T tokens,
    jb_prefill (the forward pass, fp32 o) and jb_backward (every gradient, from a random dO),
    each averaged over `reps` calls bracketed by HIP events on the launching stream."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    sh = inputs.Shape(B=B, T=T, H=sp.H, dk=sp.dk, dv=sp.dv, d_model=sp.d_model)
    p = inputs.prefill_inputs(sh, seed=9, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(10)
    dout = torch.randn((B, T, sh.H, sh.dv), generator=g, device=dev)
    shape = jb.make_shape(B, T, sh.H, sh.dk, sh.dv, sh.d_model)
    fws = jb.workspace(jb.prefill_workspace_size(shape), dev)
    bws = jb.workspace(jb.backward_workspace_size(shape), dev)
    o = torch.empty((B, T, sh.H, sh.dv), dtype=torch.float32, device=dev)
    S = torch.empty((B, sh.H, sh.dk, sh.dv), dtype=torch.float32, device=dev)

    def timed(fn, n=reps):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    ms_f = timed(lambda: jb.prefill(p["x"], p["q"], p["k"], p["v"], p["alpha"], p["beta"], p["W1"], p["W2"],
                                    o=o, S_final=S, want_conv_out=False, ws=fws, stream=stream))
    ms_b = timed(lambda: jb.backward(p["x"], p["q"], p["k"], p["v"], p["alpha"], p["beta"], p["W1"], p["W2"], dout,
                                     ws=bws, stream=stream))
    tok = B * T
    return dict(B=B, T=T, tokens=tok, forward=dict(call="jb_prefill (fp32 o)", ms=round(ms_f, 3)),
                backward=dict(call="jb_backward (all gradients)", ms=round(ms_b, 3),
                              tokens_per_s=round(tok / (ms_b * 1e-3), 1)),
                tokens_per_s=round(tok / ((ms_f + ms_b) * 1e-3), 1), backward_over_forward=round(ms_b / ms_f, 2))


def measure_4b(jb, inputs, torch, out_dt, out_bytes: int, reps: int = 3, dsteps: int = 32):
    """The JetBlock-4B-shape workload as one chain: jb_prefill of B=1, T=262144, H=16, dk=128,
    dv=256, d_model=2048 (HIP events around each call), then jb_decode_step on a batch of 128
    sequences started from the prefill's final state and conv cache (events around each
    launch), with the layer's own generator weights."""
    sp, sd = inputs.B4_T262144, inputs.B4_DECODE
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    p = inputs.prefill_inputs(sp, seed=0, device=dev)
    o = torch.empty((sp.B, sp.T, sp.H, sp.dv), dtype=out_dt, device=dev)
    S_fin = torch.empty((sp.B, sp.H, sp.dk, sp.dv), dtype=torch.float32, device=dev)
    conv_out = torch.empty((sp.B, 3, sp.H, sp.dv), dtype=torch.bfloat16, device=dev)
    shp = jb.make_shape(sp.B, sp.T, sp.H, sp.dk, sp.dv, sp.d_model, jb.JB_BF16,
                        jb.JB_BF16 if out_dt == torch.bfloat16 else jb.JB_F32)
    ws = jb.workspace(jb.prefill_workspace_size(shp), dev)

    def pre():
        jb.prefill(p["x"], p["q"], p["k"], p["v"], p["alpha"], p["beta"], p["W1"], p["W2"], out_dtype=out_dt,
                   o=o, S_final=S_fin, conv_out=conv_out, ws=ws, stream=stream)

    pre()
    torch.cuda.synchronize()
    ev = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        pre()
        e1.record(stream)
        ev.append((e0, e1))
    torch.cuda.synchronize()
    pre_ms = sum(a.elapsed_time(b) for a, b in ev) / reps

    d = inputs.decode_inputs(sd, steps=dsteps, seed=1, device=dev, with_state=False)
    S = S_fin.expand(sd.B, -1, -1, -1).contiguous()
    cache = conv_out.expand(sd.B, -1, -1, -1).contiguous()
    od = torch.empty((sd.B, sd.H, sd.dv), dtype=out_dt, device=dev)

    def dec(t):
        jb.decode_step(S, cache, d["x"][t], d["q"][t], d["k"][t], d["v"][t], d["alpha"][t], d["beta"][t],
                       p["W1"], p["W2"], out_dtype=out_dt, o=od, stream=stream)

    dec(0)
    torch.cuda.synchronize()
    ev = []
    for t in range(1, dsteps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dec(t)
        e1.record(stream)
        ev.append((e0, e1))
    torch.cuda.synchronize()
    dec_ms = sum(a.elapsed_time(b) for a, b in ev) / len(ev)
    pre_flops = prefill_flops_per_token(sp) * sp.T
    pre_tf = pre_flops / (pre_ms * 1e-3) / 1e12
    pre_gbs = prefill_bytes_per_token(sp, out_bytes) * sp.T / (pre_ms * 1e-3) / 1e9
    dec_bytes = decode_step_bytes(sd, out_bytes)
    dec_gbs = dec_bytes / (dec_ms * 1e-3) / 1e9
    out = dict(
        workload="JetBlock-4B shape: prefill B=1 T=262144 H=16 dk=128 dv=256 d_model=2048, then decode of "
                 f"B=128 from its state ({dsteps - 1} timed steps)",
        prefill=dict(ms=round(pre_ms, 4), tokens_per_s=round(sp.T / (pre_ms * 1e-3), 1),
                     roofline=dict(call="jb_prefill", bound="mfma", achieved=round(pre_tf, 2),
                                   peak=MFMA_PEAK_TFLOPS, unit="TFLOP/s", frac=round(pre_tf / MFMA_PEAK_TFLOPS, 4),
                                   hbm_GBs=round(pre_gbs, 1), hbm_frac=round(pre_gbs / HBM_PEAK_GBS, 4),
                                   flops_per_call=pre_flops)),
        decode=dict(launch_us=round(dec_ms * 1e3, 2), tokens_per_s=round(sd.B / (dec_ms * 1e-3), 1),
                    roofline=dict(kernel="decode_seq_kernel (jb_decode_step)", bound="hbm",
                                  achieved=round(dec_gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                                  frac=round(dec_gbs / HBM_PEAK_GBS, 4), bytes_per_launch=dec_bytes)))
    del p, o, ws, S, cache, d
    torch.cuda.empty_cache()
    return out


def cpu_baseline(shape_p, shape_d, prefill_tokens_per_step, decode_tokens_per_step, budget_tokens):
    """Time the fp64 oracle on a bounded sample and scale to the step's token mix."""
    import oracle
    from gated_delta_rule_jetblock_amd import inputs

    threads = min(16, len(os.sched_getaffinity(0)))
    tp = budget_tokens
    ps = shape_p.with_(T=tp)
    p = inputs.prefill_inputs(ps, seed=0)
    f = lambda t: t.float().numpy()
    args = [f(p[k]) for k in ("x", "q", "k", "v", "alpha", "beta", "W1", "W2")]
    oracle.build()
    t0 = time.perf_counter()
    oracle.prefill(*args, nthreads=threads)
    t_pre = time.perf_counter() - t0
    dsteps = 4
    d = inputs.decode_inputs(shape_d, steps=dsteps, seed=0)
    S, c = f(d["S"]), f(d["cache"])
    t0 = time.perf_counter()
    for t in range(dsteps):
        r = oracle.decode_step(S, c, *(f(d[k][t]) for k in ("x", "q", "k", "v", "alpha", "beta")), f(d["W1"]),
                               f(d["W2"]), nthreads=threads)
        S, c = r["S"].astype("float32"), r["cache"]
    t_dec = time.perf_counter() - t0
    pre_rate = tp / t_pre
    dec_rate = shape_d.B * dsteps / t_dec
    step_s = prefill_tokens_per_step / pre_rate + decode_tokens_per_step / dec_rate
    # the same oracle on one thread, on a smaller sample
    tp1 = max(256, budget_tokens // 16)
    args1 = [f(p[k][:, :tp1].contiguous()) if k in ("x", "q", "k", "v", "alpha", "beta") else f(p[k])
             for k in ("x", "q", "k", "v", "alpha", "beta", "W1", "W2")]
    t0 = time.perf_counter()
    oracle.prefill(*args1, nthreads=1)
    t_pre1 = time.perf_counter() - t0
    S, c = f(d["S"]), f(d["cache"])
    t0 = time.perf_counter()
    oracle.decode_step(S, c, *(f(d[k][0]) for k in ("x", "q", "k", "v", "alpha", "beta")), f(d["W1"]), f(d["W2"]),
                       nthreads=1)
    t_dec1 = time.perf_counter() - t0
    step1 = prefill_tokens_per_step * t_pre1 / tp1 + decode_tokens_per_step * t_dec1 / shape_d.B
    return dict(value=(prefill_tokens_per_step + decode_tokens_per_step) / step_s, unit="tokens/s", cores=threads,
                kind="oracle",
                sample=f"fp64 oracle: prefill of {tp} tokens (all {shape_p.H} heads) in {t_pre:.2f} s and "
                       f"{dsteps} decode steps x {shape_d.B} sequences in {t_dec:.2f} s, scaled to one step",
                prefill_tokens_per_s=pre_rate, decode_tokens_per_s=dec_rate,
                single_thread=dict(value=(prefill_tokens_per_step + decode_tokens_per_step) / step1, cores=1,
                                   sample=f"prefill of {tp1} tokens in {t_pre1:.2f} s and one decode step x "
                                          f"{shape_d.B} sequences in {t_dec1:.2f} s, scaled to one step"))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", choices=["2b", "4b"], default="2b")
    ap.add_argument("--out-dtype", choices=["bf16", "f32"], default="bf16")
    ap.add_argument("--decode-steps", type=int, default=128)
    ap.add_argument("--event-every", type=int, default=16,
                    help="bracket every N-th decode state-update launch with HIP events")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-from-x", action="store_true", help="skip the measurement of the block from x")
    ap.add_argument("--no-static", action="store_true", help="skip the static-conv block measurement")
    ap.add_argument("--no-serving", action="store_true", help="skip the packed serving-batch measurement")
    ap.add_argument("--no-training", action="store_true", help="skip the forward + backward measurement")
    ap.add_argument("--no-4b", action="store_true", help="skip the JetBlock-4B-shape chain (with --workload 2b)")
    ap.add_argument("--serving-requests", type=int, default=256)
    ap.add_argument("--cpu-tokens", type=int, default=16384, help="oracle prefill sample length")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run three plain 256 MiB device-to-device copies, whose counter "
                         "readings scale the HBM-traffic counters of a profiled run")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from gated_delta_rule_jetblock_amd import inputs, jetblock as jb

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload == "2b":
        sp, sd = inputs.B2_T65536, inputs.B2_DECODE
        wname = "JetBlock-2B shape: prefill B=1 T=65536 + decode B=256 x 128 steps"
    else:
        sp, sd = inputs.B4_T262144, inputs.B4_DECODE
        wname = "JetBlock-4B shape: prefill B=1 T=262144 + decode B=128 x 128 steps"
    out_dt = torch.bfloat16 if args.out_dtype == "bf16" else torch.float32
    out_bytes = 2 if args.out_dtype == "bf16" else 4
    nsteps_dec = args.decode_steps

    log(f"generating inputs on {dev} ...")
    p = inputs.prefill_inputs(sp, seed=0, device=dev)
    d = inputs.decode_inputs(sd, steps=nsteps_dec, seed=1, device=dev)
    o = torch.empty((sp.B, sp.T, sp.H, sp.dv), dtype=out_dt, device=dev)
    S_fin = torch.empty((sp.B, sp.H, sp.dk, sp.dv), dtype=torch.float32, device=dev)
    conv_out = torch.empty((sp.B, 3, sp.H, sp.dv), dtype=torch.bfloat16, device=dev)
    shp = jb.make_shape(sp.B, sp.T, sp.H, sp.dk, sp.dv, sp.d_model, jb.JB_BF16,
                        jb.JB_BF16 if out_dt == torch.bfloat16 else jb.JB_F32)
    ws = jb.workspace(jb.prefill_workspace_size(shp), dev)
    S = d["S"]
    cache = d["cache"]
    od = torch.empty((sd.B, sd.H, sd.dv), dtype=out_dt, device=dev)
    stream = torch.cuda.current_stream()

    ev_pre = []
    ev_dec = []

    def one_step(record: bool):
        if record:
            e0 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
        jb.prefill(p["x"], p["q"], p["k"], p["v"], p["alpha"], p["beta"], p["W1"], p["W2"], out_dtype=out_dt,
                   o=o, S_final=S_fin, conv_out=conv_out, ws=ws, stream=stream)
        if record:
            e1 = torch.cuda.Event(enable_timing=True)
            e1.record(stream)
            ev_pre.append((e0, e1))
        for t in range(nsteps_dec):
            rec_t = record and t % args.event_every == 0
            if rec_t:
                a0 = torch.cuda.Event(enable_timing=True)
                a0.record(stream)
            jb.decode_step(S, cache, d["x"][t], d["q"][t], d["k"][t], d["v"][t], d["alpha"][t], d["beta"][t],
                           d["W1"], d["W2"], out_dtype=out_dt, o=od, stream=stream)
            if rec_t:
                a1 = torch.cuda.Event(enable_timing=True)
                a1.record(stream)
                ev_dec.append((a0, a1))

    log(f"warmup {args.warmup} steps ...")
    for _ in range(args.warmup):
        one_step(False)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps ...")
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        one_step(True)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps
    pre_ms = sum(a.elapsed_time(b) for a, b in ev_pre) / len(ev_pre)
    dec_ms = sum(a.elapsed_time(b) for a, b in ev_dec) / len(ev_dec)
    log(f"step {ms_step:.3f} ms: prefill {pre_ms:.3f} ms, decode step {dec_ms * 1e3:.1f} us x {nsteps_dec}")

    tok_pre = sp.B * sp.T
    tok_dec = sd.B * nsteps_dec
    value = (tok_pre + tok_dec) / (ms_step * 1e-3)

    # decode step: the dominant kernel of the step
    dec_bytes = decode_step_bytes(sd, out_bytes)
    dec_gbs = dec_bytes / (dec_ms * 1e-3) / 1e9
    traffic = (measured_traffic("decode_step_jetblock2b_B256.md",
                                ["gated_delta_rule_jetblock_amd/csrc/jb_decode.hip",
                                 "gated_delta_rule_jetblock_amd/csrc/jb_device.h"])
               if args.workload == "2b" and args.out_dtype == "bf16" else None)
    roof = dict(kernel="decode_seq_kernel (jb_decode_step)", bound="hbm", achieved=round(dec_gbs, 1),
                peak=HBM_PEAK_GBS, unit="GB/s", frac=round(dec_gbs / HBM_PEAK_GBS, 4), traffic=traffic,
                bytes_per_launch=dec_bytes, avg_launch_us=round(dec_ms * 1e3, 2))
    pre_flops = prefill_flops_per_token(sp) * tok_pre
    pre_tf = pre_flops / (pre_ms * 1e-3) / 1e12
    pre_gbs = prefill_bytes_per_token(sp, out_bytes) * tok_pre / (pre_ms * 1e-3) / 1e9
    pre_traffic = (measured_traffic("prefill_jetblock2b_T65536.md",
                                    ["gated_delta_rule_jetblock_amd/csrc/jb_fwd.hip",
                                     "gated_delta_rule_jetblock_amd/csrc/jb_frag.h",
                                     "gated_delta_rule_jetblock_amd/csrc/jb_chunk.h",
                                     "gated_delta_rule_jetblock_amd/csrc/jb_device.h",
                                     "gated_delta_rule_jetblock_amd/csrc/jb_gen.hip",
                                     "gated_delta_rule_jetblock_amd/csrc/jb_prefill.hip"])
                   if args.workload == "2b" and args.out_dtype == "bf16" else None)
    roof_pre = dict(call="jb_prefill (generator, fused summary pass, segment scan, fused output pass)", bound="mfma",
                    traffic=pre_traffic, compulsory_bytes=prefill_bytes_per_token(sp, out_bytes) * tok_pre,
                    achieved=round(pre_tf, 2), peak=MFMA_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(pre_tf / MFMA_PEAK_TFLOPS, 4), hbm_GBs=round(pre_gbs, 1),
                    hbm_frac=round(pre_gbs / HBM_PEAK_GBS, 4), flops_per_call=pre_flops,
                    avg_call_ms=round(pre_ms, 4))
    from_x = None
    if not args.no_from_x:
        log("timing the block from its layer input x ...")
        from_x = measure_from_x(jb, inputs, torch, sp, out_dt)
        log(f"from x: {from_x['ms']:.3f} ms per prefill, projections {from_x['project']['ms']:.3f} ms "
            f"({from_x['project']['frac'] * 100:.1f}% of the MFMA peak), decode step from x "
            f"{from_x['decode_step_from_x']['us']:.1f} us")
    static = None
    if not args.no_static:
        log("timing the static-conv block ...")
        static = measure_static(jb, inputs, torch, sp, sd, p, d, out_dt)
        static["prefill"]["jetblock_over_static"] = round(pre_ms / static["prefill"]["ms"], 3)
        static["decode"]["jetblock_over_static"] = round(dec_ms * 1e3 / static["decode"]["us"], 3)
        log(f"static conv: prefill {static['prefill']['ms']:.3f} ms (JetBlock {pre_ms:.3f} ms), decode step "
            f"{static['decode']['us']:.1f} us (JetBlock {dec_ms * 1e3:.1f} us)")
    serving = None
    if not args.no_serving:
        log(f"timing a serving batch of {args.serving_requests} requests ...")
        serving = measure_serving(jb, inputs, torch, sp, sd, out_dt, args.serving_requests, 2048, 8192)
        log(f"serving: {serving['tokens']} prompt tokens prefilled in {serving['prefill']['ms']:.2f} ms "
            f"({serving['prefill']['tokens_per_s'] / 1e6:.1f} M tokens/s), decode step of the batch "
            f"{serving['decode']['us']:.1f} us")
    training = None
    if not args.no_training:
        log("timing forward + backward (16 x 4096 tokens) ...")
        training = measure_training(jb, inputs, torch, sp, 16, 4096)
        log(f"training: forward {training['forward']['ms']:.2f} ms, backward {training['backward']['ms']:.2f} ms "
            f"({training['tokens_per_s'] / 1e6:.2f} M tokens/s forward + backward)")
    jb4 = None
    if args.workload == "2b" and not args.no_4b:
        log("timing the JetBlock-4B-shape chain (prefill T=262144, decode B=128) ...")
        jb4 = measure_4b(jb, inputs, torch, out_dt, out_bytes)
        log(f"4B: prefill {jb4['prefill']['ms']:.3f} ms ({jb4['prefill']['roofline']['frac'] * 100:.1f}% of the "
            f"MFMA peak), decode launch {jb4['decode']['launch_us']:.1f} us "
            f"({jb4['decode']['roofline']['frac'] * 100:.1f}% of HBM)")
    if args.calibrate_copy:
        src = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device=dev)   # 256 MiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(sp, sd, tok_pre, tok_dec, args.cpu_tokens)
        log(f"cpu oracle {cpu['value']:.1f} tokens/s on {cpu['cores']} threads")

    line = {
        "metric": "JetBlock tokens/s: prefill @T=64K (%MFMA peak) + decode B=256 (%HBM peak)",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 I/O; fp16 MFMA operands, fp32 accumulate and state" if args.out_dtype == "bf16"
        else "bf16 inputs, fp32 o; fp16 MFMA operands, fp32 accumulate and state",
        "data": "synthetic (seeded)",
        "config": {"workload": wname,
                   "prefill": dict(B=sp.B, T=sp.T, H=sp.H, dk=sp.dk, dv=sp.dv, d_model=sp.d_model, chunk=64,
                                   out=args.out_dtype),
                   "decode": dict(B=sd.B, steps=nsteps_dec, H=sd.H, dk=sd.dk, dv=sd.dv, d_model=sd.d_model)},
        "prefill": dict(tokens_per_s=round(tok_pre / (pre_ms * 1e-3), 1), ms=round(pre_ms, 4),
                        mfma_frac=roof_pre["frac"], hbm_frac=roof_pre["hbm_frac"]),
        "decode": dict(tokens_per_s=round(tok_dec / ((ms_step - pre_ms) * 1e-3), 1),
                       launch_us=round(dec_ms * 1e3, 2), step_us=round((ms_step - pre_ms) / nsteps_dec * 1e3, 2),
                       hbm_frac=roof["frac"]),
        "roofline": roof,
        "roofline_prefill": roof_pre,
        "cpu_baseline": cpu,
        "from_x": from_x,
        "static_conv": static,
        "serving": serving,
        "training": training,
        "jetblock4b": jb4,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
