"""Benchmark of the KDA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-variants]
                    [--no-context] [--only prefill|decode|backward|context]

Prefill: kda_chunk_fwd on the packed-sequence workload B=1, H=16, T=4096,
dk=dv=128, chunk=64, bf16 I/O, fp32 state, zero initial state, final state
written.  Decode: kda_decode_step on B=256 sequences x H=32 heads, d=128,
against a 512 MiB resident fp32 state pool, updated in place.  Inputs are the
seeded synthetic workloads of gated_delta_rule_08_amd.workloads, already
resident in HBM before timing starts.

Each timed step is one prefill pass (then, in its own loop, one decode step).
Before every timed step a 1 GiB fill evicts the 256 MB Infinity Cache, so
inputs come from HBM; the fill is outside the HIP events that time the step.
Each leg runs its W warm-up steps, continued until the GPU has been busy with
them for 0.1 s (its clocks climb over the first tens of milliseconds of work).
`value` is prefill tokens/s = T / (mean event time of one kda_chunk_fwd call);
decode steps/s is reported next to it with its own roofline.  The oracle
(fp64, host threads) is timed on the same prefill input as a CPU baseline.

The variant flags (scalar gate, no gate, additive write) and the prefill from raw
bf16 projections (input preparation fused in) are timed on the same prefill
shape and reported under "variants", each with its own algorithmic bytes.  The
backward is timed on the same shape ("backward").  The long-context shape
(B=2, H=32, T=65,536) and the packed-varlen shape (64 sequences of 128-8,192
tokens, H=16) are timed last ("context"), each with its path roofline and the
roofline of its dominant launch.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s (H=16,d=128,T=4096) + decode steps/s; % of MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
PREFILL_BYTES_PER_TOKEN_HEAD = 3 * 2 * 128 + 4 * 128 + 4 + 2 * 128   # q,k,v bf16 + g fp32 + beta + o bf16
DECODE_BYTES_PER_HEAD = 2 * 128 * 128 * 4 + PREFILL_BYTES_PER_TOKEN_HEAD  # state read+write + token
# Algorithmic bytes of each launch of the prefill call, per token-head: the prep reads the
# inputs (q, k, v bf16, g fp32, beta), the scan writes o and the final state (per
# sequence-head, added where it is used).
PREFILL_LAUNCH_BYTES_PER_TOKEN_HEAD = {"prep_kernel": 3 * 2 * 128 + 4 * 128 + 4,
                                       "scan_out_kernel": 2 * 128}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
TRAFFIC_BACKWARD_FILE = os.path.join(ROOT, "profiles", "traffic_backward.json")


def _code_text(src: str) -> str:
    """The source with its comments removed and its whitespace collapsed: what the
    compiler sees, so that an edit of a comment keeps the digest."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def _source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_delta_rule_08_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + _code_text(f.read()).encode())
    return h.hexdigest()[:16]


def _traffic(kind: str, path: str = TRAFFIC_FILE):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None
    when the kernel sources changed since they were taken."""
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_digest") != _source_digest():
        return None
    return rec.get(kind)


def _kernel_traffic(name: str, path: str = TRAFFIC_FILE):
    """HBM bytes (fetch + write) per dispatch of one kernel from the committed counter runs,
    or None when the kernel sources changed since they were taken."""
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_digest") != _source_digest():
        return None
    for kname, k in rec.get("per_kernel", {}).items():
        if kname == name or kname.startswith(name + "<"):   # template arguments in the trace
            return k["fetch_bytes"] + k["write_bytes"]
    return None


def _events_ms(pairs):
    return [s.elapsed_time(e) for s, e in pairs]


# The GPU's clocks climb over the first tens of milliseconds of work after an idle spell
# (such as the host-side input generation before each leg): measured on the c1 prefill,
# the first 50 evicted calls after 0.2 s of idle ran 107 -> 91 us, while calls that
# follow continuous work run at 91 us from the first.  Every leg therefore keeps the GPU
# busy with its own call for at least this long before the timed steps.
SETTLE_S = 0.1


def _warm(torch, step, flush, warmup):
    """`warmup` untimed steps (each after an eviction), continued until the GPU has been
    busy with them for SETTLE_S; the host stays at most 8 calls ahead of the GPU."""
    t0 = time.perf_counter()
    n = 0
    while n < warmup or time.perf_counter() - t0 < SETTLE_S:
        flush()
        step()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def _launch_times(kda, stream, step, steps, flush):
    """Per-launch durations (ms) of `steps` calls, each after an eviction, from HIP events
    that the library records on `stream` after each of its launches."""
    times = {}
    for _ in range(steps):
        flush()
        with kda.launch_timer(stream) as lt:
            step()
        for name, ms in lt.launches:
            times.setdefault(name, []).append(ms)
    return times


def _launch_table(times, bytes_of, traffic_file):
    """{kernel: mean duration, algorithmic bytes and rate, counter traffic} from _launch_times."""
    table = {}
    for name, ms in times.items():
        mean_ms = sum(ms) / len(ms)
        b = bytes_of.get(name)
        table[name] = {"mean_us": mean_ms * 1e3, "calls": len(ms),
                       "algorithmic_bytes": b,
                       "achieved_gbs": None if b is None else b / (mean_ms * 1e-3) / 1e9,
                       "traffic": _kernel_traffic(name, traffic_file)}
    return table


def bench_prefill(kda, torch, steps, warmup, flush):
    from gated_delta_rule_08_amd import workloads
    p = workloads.make_inputs(1)
    cfg = p["config"]
    dev = "cuda"
    t = lambda a, dt: torch.from_numpy(a).to(dt).to(dev)
    q, k, v = (t(p[n], torch.bfloat16) for n in ("q", "k", "v"))
    g, beta = t(p["g"], torch.float32), t(p["beta"], torch.float32)
    cu = t(p["cu_seqlens"], torch.int32)
    T, H, d = q.shape
    N = cu.numel() - 1
    states = torch.zeros((N, H, d, d), dtype=torch.float32, device=dev)
    o = torch.empty((T, H, d), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(kda.kda_chunk_fwd_workspace_bytes(H, d, d, torch.bfloat16, cfg.chunk, T, N),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        kda.kda_chunk_fwd(q, k, v, g, beta, cu, chunk=cfg.chunk, states=states, write_final=True,
                          o=o, workspace=ws, stream=stream)

    _warm(torch, step, flush, warmup)
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(steps)]
    t0 = time.perf_counter()
    for s, e in pairs:
        flush()
        s.record(stream)
        step()
        e.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = _events_ms(pairs)
    # warm-cache figure (no eviction between steps), for context only
    ws_pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(steps)]
    for s, e in ws_pairs:
        s.record(stream)
        step()
        e.record(stream)
    torch.cuda.synchronize()
    ms_warm = _events_ms(ws_pairs)
    # per-launch durations (a separate pass: the timer adds an event after each launch)
    launches = _launch_times(kda, stream, step, steps, flush)
    return dict(cfg=cfg, T=T, H=H, d=d, N=N, ms=ms, ms_warm=ms_warm, wall=wall, inputs=p,
                launches=launches)


# Variants of the same path on the c1 shape: (flag arguments, bytes per token-head)
VARIANTS = {
    "gated_deltanet_scalar_gate": (dict(gate="scalar"), 3 * 2 * 128 + 4 + 4 + 2 * 128),
    "deltanet_no_gate": (dict(gate="none"), 3 * 2 * 128 + 4 + 2 * 128),
    "gated_linear_attention_additive": (dict(additive=True), 3 * 2 * 128 + 4 * 128 + 2 * 128),
    # raw bf16 projections: q, k, v, gate logits (bf16 per channel), write-strength logit, o
    "kda_fused_input_preparation": (dict(raw=True), 3 * 2 * 128 + 2 * 128 + 2 + 2 * 128),
}


def bench_variants(kda, torch, steps, warmup, flush):
    """Prefill tokens/s of the variant flags on the c1 shape (same timing rules)."""
    from gated_delta_rule_08_amd import workloads
    p = workloads.make_inputs(1)
    cfg = p["config"]
    t = lambda a, dt: torch.from_numpy(a).to(dt).to("cuda")
    q, k, v = (t(p[n], torch.bfloat16) for n in ("q", "k", "v"))
    g, beta = t(p["g"], torch.float32), t(p["beta"], torch.float32)
    cu = t(p["cu_seqlens"], torch.int32)
    T, H, d = q.shape
    N = cu.numel() - 1
    g_scalar = g[..., 0].contiguous()      # one log-decay per (token, head)
    # raw projections of the same shape (the prep normalises q, k and squashes the logits)
    gen = torch.Generator(device="cuda").manual_seed(1001)
    q_raw = torch.randn(q.shape, device="cuda", generator=gen).to(torch.bfloat16)
    k_raw = torch.randn(k.shape, device="cuda", generator=gen).to(torch.bfloat16)
    a_raw = (torch.randn(g.shape, device="cuda", generator=gen) + 3.0).to(torch.bfloat16)
    b_raw = torch.randn(beta.shape, device="cuda", generator=gen).to(torch.bfloat16)
    states = torch.zeros((N, H, d, d), dtype=torch.float32, device="cuda")
    o = torch.empty((T, H, d), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(kda.kda_chunk_fwd_workspace_bytes(H, d, d, torch.bfloat16, cfg.chunk, T, N),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    out = {}
    for name, (kw, per_token_head) in VARIANTS.items():
        gate = kw.get("gate", "channel")
        gg = {"channel": g, "scalar": g_scalar, "none": None}[gate]
        bb = None if kw.get("additive") else beta

        def step():
            if kw.get("raw"):
                kda.kda_chunk_fwd_raw(q_raw, k_raw, v, a_raw, b_raw, cu, chunk=cfg.chunk,
                                      states=states, write_final=True, o=o, workspace=ws,
                                      stream=stream)
            else:
                kda.kda_chunk_fwd(q, k, v, gg, bb, cu, chunk=cfg.chunk, states=states,
                                  write_final=True, o=o, workspace=ws, stream=stream, **kw)

        _warm(torch, step, flush, warmup)
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(steps)]
        for s_, e_ in pairs:
            flush()
            s_.record(stream)
            step()
            e_.record(stream)
        torch.cuda.synchronize()
        ms = sum(_events_ms(pairs)) / steps
        bytes_ = per_token_head * T * H + N * H * d * d * 4
        out[name] = {"tokens_per_s": T / (ms * 1e-3), "ms_per_call": ms,
                     "algorithmic_bytes": bytes_,
                     "roofline_frac": bytes_ / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    return out


# Backward on the c1 shape: reads q, k, v, g, beta, dO; writes dq, dk, dv, dg, dbeta.
BACKWARD_BYTES_PER_TOKEN_HEAD = (3 * 2 * 128 + 4 * 128 + 4 + 2 * 128) + (3 * 2 * 128 + 4 * 128 + 4)


def _time_calls(torch, step, steps, warmup, flush):
    """Mean HIP-event time (ms) of step() on the current stream, cache evicted before each."""
    stream = torch.cuda.current_stream()
    _warm(torch, step, flush, warmup)
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(steps)]
    for s_, e_ in pairs:
        flush()
        s_.record(stream)
        step()
        e_.record(stream)
    torch.cuda.synchronize()
    return sum(_events_ms(pairs)) / steps


def bench_backward(kda, torch, steps, warmup, flush, with_variants=True):
    """kda_chunk_bwd tokens/s on the c1 shape (same timing rules as the prefill), and the
    scalar-gate and raw-projection variants of it."""
    from gated_delta_rule_08_amd import workloads
    p = workloads.make_inputs(1)
    cfg = p["config"]
    t = lambda a, dt: torch.from_numpy(a).to(dt).to("cuda")
    q, k, v = (t(p[n], torch.bfloat16) for n in ("q", "k", "v"))
    g, beta = t(p["g"], torch.float32), t(p["beta"], torch.float32)
    cu = t(p["cu_seqlens"], torch.int32)
    T, H, d = q.shape
    N = cu.numel() - 1
    gen = torch.Generator(device="cuda").manual_seed(1002)
    do = torch.randn(q.shape, device="cuda", generator=gen).to(torch.bfloat16)
    out = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
               dg=torch.empty_like(g), dbeta=torch.empty_like(beta), d_initial=None)
    ws = torch.empty(kda.kda_chunk_bwd_workspace_bytes(H, d, d, torch.bfloat16, cfg.chunk, T, N),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        kda.kda_chunk_bwd(q, k, v, g, beta, cu, do, chunk=cfg.chunk, workspace=ws, stream=stream,
                          out=out)

    _warm(torch, step, flush, warmup)
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(steps)]
    for s_, e_ in pairs:
        flush()
        s_.record(stream)
        step()
        e_.record(stream)
    torch.cuda.synchronize()
    ms = sum(_events_ms(pairs)) / steps
    bytes_ = BACKWARD_BYTES_PER_TOKEN_HEAD * T * H
    # per launch: the prep reads the forward inputs, the paired scans read dL/do, the
    # gradient kernel writes dq, dk, dv, dg, dbeta
    launch_bytes = {"prep_kernel": (3 * 2 * 128 + 4 * 128 + 4) * T * H,
                    "scan_pair_kernel": 2 * 128 * T * H,
                    "grad_kernel": (3 * 2 * 128 + 4 * 128 + 4) * T * H}
    launches = _launch_table(_launch_times(kda, stream, step, steps, flush), launch_bytes,
                             TRAFFIC_BACKWARD_FILE)
    result = {"tokens_per_s": T / (ms * 1e-3), "ms_per_call": ms, "algorithmic_bytes": bytes_,
              "roofline_frac": bytes_ / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
              "traffic": _traffic("backward_bytes", TRAFFIC_BACKWARD_FILE),
              "launches": launches,
              "workload": "backward_bf16_B1_H16_T4096_d128_C64 (dL/do given, zero initial state)"}
    if not with_variants:
        return result
    # variants: a [T, H] gate (Gated DeltaNet); raw bf16 projections (preparation and its
    # chain rule included)
    g1 = g[..., 0].contiguous()
    ws_raw = torch.empty(kda.kda_chunk_bwd_raw_workspace_bytes(H, d, d, torch.bfloat16, cfg.chunk,
                                                               T, N),
                         dtype=torch.uint8, device="cuda")
    q_raw = torch.randn(q.shape, device="cuda", generator=gen).to(torch.bfloat16)
    k_raw = torch.randn(k.shape, device="cuda", generator=gen).to(torch.bfloat16)
    a_raw = (torch.randn(g.shape, device="cuda", generator=gen) + 3.0).to(torch.bfloat16)
    b_raw = torch.randn(beta.shape, device="cuda", generator=gen).to(torch.bfloat16)
    ms_scalar = _time_calls(torch, lambda: kda.kda_chunk_bwd(
        q, k, v, g1, beta, cu, do, chunk=cfg.chunk, workspace=ws, stream=stream, gate="scalar"),
        steps, warmup, flush)
    ms_raw = _time_calls(torch, lambda: kda.kda_chunk_bwd_raw(
        q_raw, k_raw, v, a_raw, b_raw, cu, do, chunk=cfg.chunk, workspace=ws_raw, stream=stream),
        steps, warmup, flush)
    b_scalar = (BACKWARD_BYTES_PER_TOKEN_HEAD - 2 * 4 * 127) * T * H
    # raw: reads bf16 q, k, v, dO, gate and beta logits; writes bf16 dq, dk, dv, gate, beta grads
    b_raw_ = (4 * 256 + 256 + 2 + 3 * 256 + 256 + 2) * T * H
    variants = {
        "gated_deltanet_scalar_gate": {"tokens_per_s": T / (ms_scalar * 1e-3), "ms_per_call": ms_scalar,
                                       "algorithmic_bytes": b_scalar,
                                       "roofline_frac": b_scalar / (ms_scalar * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "from_raw_projections": {"tokens_per_s": T / (ms_raw * 1e-3), "ms_per_call": ms_raw,
                                 "algorithmic_bytes": b_raw_,
                                 "roofline_frac": b_raw_ / (ms_raw * 1e-3) / 1e9 / HBM_PEAK_GBS},
    }
    result["variants"] = variants
    return result


def bench_decode(kda, torch, steps, warmup, flush):
    from gated_delta_rule_08_amd import workloads
    p = workloads.make_inputs(2)
    dev = "cuda"
    t = lambda a, dt: torch.from_numpy(a).to(dt).to(dev)
    q, k, v = (t(p[n], torch.bfloat16) for n in ("q", "k", "v"))
    g, beta = t(p["g"], torch.float32), t(p["beta"], torch.float32)
    states = t(p["s0"], torch.float32)
    B, H, d = q.shape
    o = torch.empty((B, H, d), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        kda.kda_decode_step(q, k, v, g, beta, states, o=o, stream=stream)

    _warm(torch, step, flush, warmup)
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(steps)]
    for s, e in pairs:
        flush()
        s.record(stream)
        step()
        e.record(stream)
    torch.cuda.synchronize()
    return dict(B=B, H=H, d=d, ms=_events_ms(pairs))


def cpu_baseline(p, budget_s=10.0):
    import oracle
    nthreads = min(16, os.cpu_count() or 1, p["q"].shape[1])
    T = p["q"].shape[0]
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.run(p["q"], p["k"], p["v"], p["g"], p["beta"], p["cu_seqlens"], nthreads=nthreads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or el / reps * (reps + 1) > 3 * budget_s:
            break
    return {"value": reps * T / el, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "sample": f"the full prefill input (T={T}, H={p['q'].shape[1]}, d=128), run {reps}x "
                      f"in {el:.1f} s, fp64 sequential recurrence, one thread per head"}


def bench_context(kda, torch, flush, calls=5, warmup=2):
    """Prefill on the long-context shape (2 x 65,536 tokens, 32 heads) and the packed-varlen
    shape (64 sequences of 128-8,192 tokens, 16 heads, half of them with a scalar gate,
    initial states given).  Inputs follow the generators' distributions but are drawn on the
    GPU (host generation of 8.6e8 values per tensor would dominate the run): unit-norm q and k
    rows, normal v, beta = sigmoid(normal), log alpha = log sigmoid(normal + mu); the sequence
    lengths are the generator's own.  Each call follows a cache eviction; per-launch times come
    from the library's launch timer.  Algorithmic bytes per call: 1,540 per token-head (q, k,
    v, o bf16; g fp32 per channel, the scalar-gate heads included, as the call reads it; beta)
    plus the final states written and, where given, the initial states read (64 KiB per
    sequence-head each)."""
    from gated_delta_rule_08_amd import workloads
    import numpy as np
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    nz = lambda *shape: torch.randn(*shape, device="cuda", generator=gen)
    norm = torch.nn.functional.normalize
    res = {}
    for index in (3, 4):
        cfg = workloads.CONFIGS[index]
        lens = workloads.seq_lengths(cfg)
        T, N, H, d = int(lens.sum()), len(lens), cfg.num_heads, cfg.dk
        q = norm(nz(T, H, d), dim=-1).to(torch.bfloat16)
        k = norm(nz(T, H, d), dim=-1).to(torch.bfloat16)
        v = nz(T, H, d).to(torch.bfloat16)
        beta = torch.sigmoid(nz(T, H))
        g = torch.nn.functional.logsigmoid(nz(T, H, d) + cfg.alpha_mu)
        for h in cfg.scalar_gate_heads:
            g[:, h, :] = g[:, h, :1]
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), device="cuda")
        states = (0.02 * nz(N, H, d, d)) if cfg.with_s0 else torch.zeros(N, H, d, d, device="cuda")
        ws = torch.empty(kda.kda_chunk_fwd_workspace_bytes(H, d, d, torch.bfloat16, cfg.chunk, T, N),
                         dtype=torch.uint8, device="cuda")
        o = torch.empty_like(v)
        call = lambda: kda.kda_chunk_fwd(q, k, v, g, beta, cu, chunk=cfg.chunk, states=states,
                                         read_initial=cfg.with_s0, write_final=True, o=o,
                                         workspace=ws)
        _warm(torch, call, flush, warmup)
        stream = torch.cuda.current_stream()
        ms, per = [], {}
        for _ in range(calls):
            flush()
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record(stream)
            with kda.launch_timer(stream) as lt:
                call()
            t1.record(stream)
            torch.cuda.synchronize()
            ms.append(t0.elapsed_time(t1))
            for name, x in lt.launches:
                per.setdefault(name, []).append(x)
        m = sum(ms) / len(ms)
        state_bytes = N * H * d * d * 4 * (2 if cfg.with_s0 else 1)
        bytes_ = PREFILL_BYTES_PER_TOKEN_HEAD * T * H + state_bytes
        achieved = bytes_ / (m * 1e-3) / 1e9
        # per launch: the prep reads the inputs, the scan writes o and the states
        launch_bytes = {"prep_kernel": PREFILL_LAUNCH_BYTES_PER_TOKEN_HEAD["prep_kernel"] * T * H}
        for name in per:
            if name.startswith("scan"):
                launch_bytes[name] = 2 * 128 * T * H + state_bytes
        launches = {n: {"mean_us": 1e3 * sum(x) / len(x), "calls": len(x),
                        "algorithmic_bytes": launch_bytes.get(n),
                        "achieved_gbs": (None if launch_bytes.get(n) is None else
                                         launch_bytes[n] / (1e-3 * sum(x) / len(x)) / 1e9)}
                    for n, x in per.items()}
        dom = max(launches, key=lambda n: launches[n]["mean_us"])
        dl = launches[dom]
        res[cfg.name] = {
            "tokens": T, "sequences": N, "heads": H, "ms_per_call": m,
            "tokens_per_s": T / (m * 1e-3), "calls": calls, "algorithmic_bytes": bytes_,
            "path_roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                              "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS},
            "roofline": {"bound": "hbm", "kernel": dom, "achieved": dl["achieved_gbs"],
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": (None if dl["achieved_gbs"] is None
                                  else dl["achieved_gbs"] / HBM_PEAK_GBS),
                         "algorithmic_bytes": dl["algorithmic_bytes"],
                         "duration_us": dl["mean_us"]},
            "launches": launches,
            "data": "synthetic, drawn on the GPU with the generators' distributions",
        }
        print(f"{cfg.name}: {m:.3f} ms per call", file=sys.stderr, flush=True)
        del q, k, v, g, beta, states, ws, o
        torch.cuda.empty_cache()
    return res


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the prefill timings of the variant flags")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the prefill on the long-context and packed-varlen shapes")
    ap.add_argument("--only", choices=["prefill", "decode", "backward", "context"], default=None,
                    help="run one leg only (for profiling); 'context' times the prefill on the "
                         "long-context and packed-varlen shapes instead (its own JSON line)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run one plain device copy of MIB MiB (reference for the "
                         "FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the operator shards over "
              "(sequence, head) pairs with no communication, so one GPU's share is what it "
              "measures", file=sys.stderr)
        return 2
    import torch
    import gated_delta_rule_08_amd as kda
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    kda.load_library()
    # No cyclic garbage collection while anything is timed: a full collection that falls
    # inside an event-timed region can stall the launching thread for tens of milliseconds
    # while the GPU idles (the likely cause of a 3.8 ms mean over ten 0.3 ms calls).
    gc.collect()
    gc.disable()
    flush_buf = torch.empty(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
    counter = [0]

    def flush():
        counter[0] += 1
        flush_buf.fill_(float(counter[0] & 7))

    if args.copy_calibration:
        src = torch.empty(args.copy_calibration << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1.0)
        flush()
        torch.mul(src, 1.0, out=dst)   # reads and writes exactly MIB MiB
        torch.cuda.synchronize()
        del src, dst

    if args.only == "context":
        print(json.dumps({"metric": "KDA prefill tokens/s on the long-context and packed-varlen "
                                    "shapes", "unit": "tokens/s", "n_gpus": 1,
                          "higher_is_better": True, "dtype": "bf16",
                          "data": "synthetic (drawn on the GPU)",
                          "context": bench_context(kda, torch, flush)}), flush=True)
        return 0
    out = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic"}
    if args.only in (None, "prefill"):
        pr = bench_prefill(kda, torch, args.steps, args.warmup, flush)
        ms = sum(pr["ms"]) / len(pr["ms"])
        T, H, N = pr["T"], pr["H"], pr["N"]
        bytes_ = PREFILL_BYTES_PER_TOKEN_HEAD * T * H + N * H * 128 * 128 * 4
        achieved = bytes_ / (ms * 1e-3) / 1e9
        launch_bytes = {k: b * T * H for k, b in PREFILL_LAUNCH_BYTES_PER_TOKEN_HEAD.items()}
        launch_bytes["scan_out_kernel"] += N * H * 128 * 128 * 4   # final state
        launches = _launch_table(pr["launches"], launch_bytes, TRAFFIC_FILE)
        dom = max(launches, key=lambda n: launches[n]["mean_us"])
        dl = launches[dom]
        ms_sorted = sorted(pr["ms"])
        out.update({
            "value": T / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms,
            "config": {"workload": pr["cfg"].name, "global_batch": 1, "seq_len": T,
                       "num_heads": H, "head_dim": 128, "chunk": 64, "io": "bf16",
                       "state": "fp32", "parallelism": "single-gpu"},
            # the dominant launch of the call, timed by the library's own events
            "roofline": {"bound": "hbm", "kernel": dom, "achieved": dl["achieved_gbs"],
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": dl["achieved_gbs"] / HBM_PEAK_GBS, "traffic": dl["traffic"],
                         "algorithmic_bytes": dl["algorithmic_bytes"],
                         "duration_us": dl["mean_us"]},
            # the whole call (all launches) against the path's algorithmic bytes
            "path_roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                              "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                              "traffic": _traffic("prefill_bytes"),
                              "kernel": "kda_chunk_fwd (" + ", ".join(pr["launches"]) + ")",
                              "algorithmic_bytes": bytes_},
            "launches": launches,
            "prefill_ms": {"mean": ms, "median": ms_sorted[len(ms_sorted) // 2],
                           "min": ms_sorted[0], "max": ms_sorted[-1],
                           "warm_cache_mean": sum(pr["ms_warm"]) / len(pr["ms_warm"])},
            "wall_s_timed_region": pr["wall"],
        })
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = cpu_baseline(pr["inputs"])
        del pr
        if not args.no_variants:
            out["variants"] = bench_variants(kda, torch, max(5, args.steps // 2), 2, flush)
            out["backward"] = bench_backward(kda, torch, max(5, args.steps // 2), 2, flush)
    if args.only == "backward":
        bw = bench_backward(kda, torch, args.steps, args.warmup, flush,
                            with_variants=not args.no_variants)
        out.update({"value": bw["tokens_per_s"], "unit": "tokens/s", "ms_per_step": bw["ms_per_call"],
                    "config": {"workload": bw["workload"]}, "backward": bw})
    if args.only in (None, "decode"):
        dc = bench_decode(kda, torch, args.steps, args.warmup, flush)
        ms = sum(dc["ms"]) / len(dc["ms"])
        bytes_ = DECODE_BYTES_PER_HEAD * dc["B"] * dc["H"]
        achieved = bytes_ / (ms * 1e-3) / 1e9
        out["decode"] = {
            "value": 1e3 / ms, "unit": "steps/s", "ms_per_step": ms,
            "tokens_per_s": dc["B"] * 1e3 / ms,
            "workload": "decode_bf16_B256_H32_d128 (512 MiB fp32 state pool)",
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                         "traffic": _traffic("decode_bytes"), "kernel": "decode_kernel",
                         "algorithmic_bytes": bytes_},
        }
        if args.only == "decode":
            out.update({"value": 1e3 / ms, "unit": "steps/s", "ms_per_step": ms,
                        "config": {"workload": "decode_bf16_B256_H32_d128"}})
    if args.only is None and not args.no_context:
        # the long-context and packed-varlen shapes: parity cases that also carry throughput
        out["context"] = bench_context(kda, torch, flush)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
