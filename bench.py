"""Benchmark: causal kernelized linear attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu-baseline] [--only NAME]

A step is one full forward pass of the hot path (feature map, gate prelude,
segment states, segment chaining, chunked outputs) over one batch of the
headline workload: GLA-gated causal elu+1 linear attention, B=2 H=16 n=16384
d_k=d_v=128, bf16 inputs and outputs, fp32 state, 64-token chunks (the largest
of the measured configurations). Inputs are seeded synthetic tensors already
resident in HBM; several copies at different addresses are rotated so that
consecutive steps do not find their inputs in the 256 MB last-level (MALL)
cache. Timing uses HIP events on the stream the library launches on; a second
run of the same steps brackets every kernel launch with events
(la_timing_begin / la_timing_end) for the per-kernel durations behind the
roofline. Rank 0 prints one JSON line.

The same line carries, under "extra", the other workloads (non-causal fp32,
causal elu+1, RetNet decay, the outer-product gate, the state-space forms,
FAVOR+, the GLA decode step, the serving batch and the backward passes), and
the fp64 CPU oracle (blocked form) timed on the host's cores on a bounded
sample of the headline workload. ``--only NAME`` runs one workload and prints
its record alone (for per-workload profiles).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import resource
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

from workloads import WORKLOADS, HEADLINE, make_inputs  # noqa: E402

METRIC = "causal linear-attn fwd tokens/s (B·H·n) at 1 MI355X; % MFMA peak, decode % HBM BW"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 matrix peak
MALL_BYTES = 256 << 20
CHUNK = 64


def algorithmic_per_token(wl):
    """(bytes, matrix-core flops) per head-token that the method must move/do.

    Bytes: read q, k, v (and g; the outer-product gate also gv) once, write o once. Flops (chunk C = 64, masked
    upper triangle excluded): scores (C+1)/2 * 2r, intra A.V (C+1)/2 * 2 d_v,
    inter-chunk read 2 r d_v, state update 2 r d_v, FAVOR+ projection 2 * 2 d_k r.
    """
    isz = 4 if wl.dtype == "f32" else 2
    nbytes = isz * (2 * wl.d_k + wl.d_v) + isz * wl.d_v
    if wl.gate == "gla":
        nbytes += isz * wl.r
    if wl.gate == "sel":
        nbytes += isz
    if wl.gate == "outer":
        nbytes += isz * (wl.r + wl.d_v)
    half = (CHUNK + 1) / 2
    flops = half * 2 * wl.r + half * 2 * wl.d_v + 4 * wl.r * wl.d_v
    if wl.fmap == "favor":
        flops += 2 * 2 * wl.d_k * wl.r
    if not wl.causal:
        flops = 4 * wl.r * wl.d_v
    return nbytes, flops


def source_digest():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "kernelized_sequence_mixing_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def _profile_entry(workload, kernel):
    """The committed rocprofv3 summary of `kernel` on `workload`
    (profiles/traffic_<workload>.json), if it was taken on the current kernel
    sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_digest") != source_digest():
        return None
    return t.get("kernels", {}).get(kernel)


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    rocprofv3 counter summary (FETCH_SIZE and WRITE_SIZE, calibrated on a plain
    copy), if it was taken on the current kernel sources; else None."""
    k = _profile_entry(workload, kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def measured_mfma(workload, kernel):
    """Counter-measured matrix-core use of `kernel` on `workload` from the same
    summary: issued bf16 MFMA flops (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512) per
    launch and over its traced duration, and the MFMA-busy fraction
    (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x SIMDs); else None."""
    k = _profile_entry(workload, kernel)
    if k is None or k.get("mfma_flops") is None:
        return None
    return {"kernel": k.get("kernel"), "issued_flops_per_launch": k["mfma_flops"],
            "issued_TFLOPs": k.get("mfma_tflops"), "issued_frac": k.get("mfma_frac"),
            "busy_frac": k.get("mfma_busy"), "traced_us": k.get("avg_us")}


def _device_sets(inp, keys, per_set_bytes):
    """Copies of the inputs at distinct addresses, enough to exceed 3x the MALL."""
    n_sets = max(1, math.ceil(3 * MALL_BYTES / max(per_set_bytes, 1)))
    n_sets = min(n_sets, 8)
    sets = []
    for _ in range(n_sets):
        sets.append({k: (inp[k].to("cuda", non_blocking=False).clone() if isinstance(inp.get(k), torch.Tensor) else inp.get(k))
                     for k in keys})
    return sets


def time_steps(fn, n_sets, steps, warmup, stream):
    """Mean ms per step over `steps` back-to-back steps (HIP events on `stream`
    around the whole run, device synchronised on both sides), and the median of
    a second, separately timed run with an event pair around every step (those
    events serialise the queue between steps, so the median includes that)."""
    for i in range(warmup):
        fn(i % n_sets)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        fn(i % n_sets)
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    per = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        per[i][0].record(stream)
        fn(i % n_sets)
        per[i][1].record(stream)
    torch.cuda.synchronize()
    step_ms = sorted(a.elapsed_time(b) for a, b in per)
    return total_ms / steps, step_ms[len(step_ms) // 2]


def forward_kernel_names(wl, P):
    """Kernel names of one la_forward call, in launch order."""
    if not wl.causal:
        return ["nc_partial", "nc_readout"]
    pre = "favor" if wl.fmap == "favor" else "causal"
    # the GLA gate's segment pass is the feature-major kernel where it is built (64 or 128 features)
    seg = "gla_segment_state" if (wl.gate == "gla" and wl.fmap != "favor" and wl.d_k % 64 == 0) \
        else f"{pre}_segment_state"
    return [seg, "segment_scan_kernel", f"{pre}_chunk_forward"] if P > 1 else [f"{pre}_chunk_forward"]


def kernel_table(times, names):
    """Average ms per launch index over the timed calls, labelled with `names`."""
    n = len(times[0])
    if any(len(t) != n for t in times):
        raise RuntimeError("calls made different numbers of launches")
    if len(names) != n:
        names = [f"launch{i}" for i in range(n)]
    return [{"name": names[i], "avg_ms": round(sum(t[i] for t in times) / len(times), 5),
             "min_ms": round(min(t[i] for t in times), 5)} for i in range(n)]


def bench_forward(wl, steps, warmup):
    import kernelized_sequence_mixing_amd as ksm
    inp = make_inputs(wl, seed=0)
    keys = ["Q", "K", "V", "g", "gv", "gamma", "omega"]
    nb_tok, fl_tok = algorithmic_per_token(wl)
    per_set = wl.head_tokens * nb_tok
    sets = _device_sets(inp, keys, per_set)
    gate_of = {
        "none": lambda s: None,
        "decay": lambda s: ("decay", s["gamma"]),
        "gla": lambda s: ("gla", s["g"], wl.tau),
        "sel": lambda s: ("sel", s["g"], wl.tau),
        "outer": lambda s: ("outer", s["g"], s["gv"], wl.tau),
    }[wl.gate]
    outs = [torch.empty((wl.B, wl.H, wl.n, wl.d_v), dtype=sets[0]["V"].dtype, device="cuda") for _ in sets]
    nws = ksm.workspace_size(wl.B, wl.H, wl.n, wl.d_k, wl.d_v, fmap=wl.fmap, r=wl.r, causal=wl.causal,
                             gate_kind=wl.gate, dtype=sets[0]["Q"].dtype)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    # arguments marshalled once per input set: the timed loop is one foreign call per step
    calls = [ksm.PreparedForward(s["Q"], s["K"], s["V"], fmap=wl.fmap, omega=s["omega"], causal=wl.causal,
                                 gate=gate_of(s), eps=wl.eps, out=outs[i], workspace=ws, stream=stream)
             for i, s in enumerate(sets)]

    def step(i):
        calls[i]()

    ms, med = time_steps(step, len(sets), steps, warmup, stream)
    order = iter(range(steps))
    times = ksm.launch_times(lambda: calls[next(order) % len(calls)](), steps, stream)
    P = ksm.segments(wl.B, wl.H, wl.n, wl.d_k, wl.d_v, fmap=wl.fmap, r=wl.r, causal=wl.causal,
                     gate_kind=wl.gate, dtype=sets[0]["Q"].dtype)[0] if wl.causal else 1
    tok_s = wl.head_tokens / (ms * 1e-3)
    res = {"workload": wl.name, "ms_per_step": round(ms, 5), "median_ms": round(med, 5),
           "value": tok_s, "unit": "head-tokens/s", "input_sets_rotated": len(sets),
           "segments": P, "kernels": kernel_table(times, forward_kernel_names(wl, P))}
    gbs = per_set / (ms * 1e-3) / 1e9
    tfl = wl.head_tokens * fl_tok / (ms * 1e-3) / 1e12
    res["hbm_alg_GBs"] = round(gbs, 1)
    res["hbm_frac"] = round(gbs / HBM_PEAK_GBS, 4)
    res["mfma_alg_TFLOPs"] = round(tfl, 2)
    res["mfma_frac"] = round(tfl / BF16_PEAK_TFLOPS, 4)
    res["alg_bytes_per_token"] = nb_tok
    res["alg_flops_per_token"] = fl_tok
    return res


def bench_decode(wl, steps, warmup):
    import kernelized_sequence_mixing_amd as ksm
    inp = make_inputs(wl, seed=0)
    isz = 2 if wl.dtype == "bf16" else 4
    per_head = 2 * wl.r * wl.d_v * 4 + 2 * wl.r * 4 + isz * (2 * wl.d_k + wl.d_v + wl.r) + 4 * wl.d_v
    per_step = wl.B * wl.H * per_head
    keys = ["S0", "z0", "q", "k", "v", "g"]
    sets = _device_sets(inp, keys, per_step)
    outs = [torch.empty((wl.B, wl.H, wl.d_v), dtype=torch.float32, device="cuda") for _ in sets]
    stream = torch.cuda.current_stream()

    calls = [ksm.PreparedDecode(s["S0"], s["z0"], s["q"], s["k"], s["v"], gate=("gla", s["g"], wl.tau), eps=wl.eps,
                                out=outs[i], stream=stream) for i, s in enumerate(sets)]

    def step(i):
        calls[i]()

    ms, med = time_steps(step, len(sets), steps, warmup, stream)
    gbs = per_step / (ms * 1e-3) / 1e9
    return {"workload": wl.name, "ms_per_step": round(ms, 5), "median_ms": round(med, 5),
            "value": wl.B * wl.H / (ms * 1e-3), "unit": "head-tokens/s (one decode step per head)",
            "input_sets_rotated": len(sets), "alg_bytes_per_step": per_step, "hbm_alg_GBs": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


def bench_serve_prefill(steps, warmup, num_seqs=32, H=16, d=64):
    """la_forward_batch over a ragged prefill: num_seqs sequences of a seeded
    log-uniform length mix (64 .. 8192 tokens) packed along n, causal elu+1,
    each storing its final state in its slot. Bytes per head-token as the
    headline (q, k, v read, o written) plus each sequence's stored state."""
    import kernelized_sequence_mixing_amd as ksm
    from workloads import serving_lengths
    lens = serving_lengths(num_seqs, seed=7)
    T = int(lens.sum())
    wl = WORKLOADS["causal_elu1"].resized(name="serve_prefill", B=1, H=H, n=T, d_k=d, d_v=d, r=d)
    inp = make_inputs(wl, seed=0)
    inp["cu"] = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32))
    inp["ids"] = torch.arange(num_seqs, dtype=torch.int32)
    state_bytes = num_seqs * H * (d * d + d) * 4
    per_set = H * T * 4 * 2 * d + state_bytes
    sets = _device_sets(inp, ["Q", "K", "V", "cu", "ids"], per_set)
    stream = torch.cuda.current_stream()
    pools = [(torch.empty((num_seqs, H, d, d), dtype=torch.float32, device="cuda"),
              torch.empty((num_seqs, H, d), dtype=torch.float32, device="cuda")) for _ in sets]
    calls = [ksm.PreparedForwardBatch(s["Q"], s["K"], s["V"], cu_seqlens=s["cu"], max_seqlen=int(lens.max()),
                                      state=pools[i], slot_ids=s["ids"], write=True, eps=wl.eps, stream=stream)
             for i, s in enumerate(sets)]
    ms, med = time_steps(lambda i: calls[i](), len(sets), steps, warmup, stream)
    gbs = per_set / (ms * 1e-3) / 1e9
    return {"workload": "serve_prefill_ragged", "ms_per_step": round(ms, 5), "median_ms": round(med, 5),
            "value": H * T / (ms * 1e-3), "unit": "head-tokens/s", "input_sets_rotated": len(sets),
            "hbm_alg_GBs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "alg_bytes_per_step": per_set,
            "shape": {"num_seqs": num_seqs, "tokens": T, "H": H, "d_k": d, "d_v": d, "min_len": int(lens.min()),
                      "max_len": int(lens.max()), "gate": "none", "feature_map": "elu+1"}}


def bench_serve_decode(wl, m, steps, warmup):
    """la_forward_batch as a decode step of m tokens for each of B sequences
    (the GLA decode configuration), every sequence reading and writing its
    state slot in place. Bytes per step: each head's state read and written,
    plus m tokens of q, k, v, g read and o written."""
    import kernelized_sequence_mixing_amd as ksm
    B, H, r, dv, dk = wl.B, wl.H, wl.r, wl.d_v, wl.d_k
    base = WORKLOADS["gla_gate"].resized(name=f"serve_decode_m{m}", B=B, H=H, n=m)
    inp = make_inputs(base, seed=0)
    dec = make_inputs(wl, seed=0)
    inp["S"], inp["z"] = dec["S0"], dec["z0"]
    inp["ids"] = torch.arange(B, dtype=torch.int32)
    per_head = 2 * (r * dv + r) * 4 + m * 2 * (2 * dk + dv + r) + m * 2 * dv
    per_step = B * H * per_head
    sets = _device_sets(inp, ["Q", "K", "V", "g", "S", "z", "ids"], per_step)
    stream = torch.cuda.current_stream()
    calls = [ksm.PreparedForwardBatch(s["Q"], s["K"], s["V"], state=(s["S"], s["z"]), slot_ids=s["ids"], read=True,
                                      write=True, gate=("gla", s["g"], wl.tau), eps=wl.eps, stream=stream)
             for s in sets]
    ms, med = time_steps(lambda i: calls[i](), len(sets), steps, warmup, stream)
    gbs = per_step / (ms * 1e-3) / 1e9
    return {"workload": f"serve_decode_slots_m{m}", "ms_per_step": round(ms, 5), "median_ms": round(med, 5),
            "value": B * H * m / (ms * 1e-3), "unit": "head-tokens/s", "input_sets_rotated": len(sets),
            "alg_bytes_per_step": per_step, "hbm_alg_GBs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "shape": {"B": B, "H": H, "m": m, "r": r, "d_v": dv, "gate": "gla"}}


def backward_algorithmic_per_token(wl):
    """(bytes, matrix-core flops) per head-token of the backward pass (causal unless wl.causal is False).

    Bytes: read q, k, v, dO once, write dq, dk, dv once (GLA: also read g and
    write dg, r per token each; the selective gate: one of each per token; the
    outer-product gate: g and dg, plus gv and dgv, d_v per token each). Flops
    (chunk C, masked upper triangle excluded): the scores, the
    numerator of o, dW, and the intra-chunk parts of dq, dk, dv ((C+1)/2 * 2 r
    or 2 d_v each), plus six r x d_v products per token (o's inter-chunk read,
    dq's S g, dk's R v, dv's R phi(k), and the forward and reverse state
    updates).
    """
    isz = 4 if wl.dtype == "f32" else 2
    nbytes = isz * (2 * wl.d_k + 2 * wl.d_v) + isz * (2 * wl.d_k + wl.d_v)
    if wl.gate == "gla":
        nbytes += 2 * (2 * wl.r)
    elif wl.gate == "sel":
        nbytes += 2 * 2
    elif wl.gate == "outer":
        nbytes += 2 * (2 * wl.r) + 2 * (2 * wl.d_v)
    half = (CHUNK + 1) / 2
    flops = half * 2 * wl.r * 3 + half * 2 * wl.d_v * 3 + 6 * 2 * wl.r * wl.d_v
    if not wl.causal:  # the non-causal form: S, G and the per-token products, no scores
        flops = 6 * 2 * wl.r * wl.d_v
    if wl.fmap == "favor":  # phi(q), phi(k) and their pullbacks: four r x d_k products per token
        flops += 4 * 2 * wl.r * wl.d_k
    return nbytes, flops


def backward_kernel_names(wl, count):
    """Labels of la_backward's launches, in order: with several segments the forward's
    segment-state pass and scan, pass A, the reverse state pass and reverse scan, pass B
    (one segment: A and B only); 128 x 128 states repeat them per value-column half;
    FAVOR+ adds the feature kernels before and the pullbacks through the map after."""
    favor = wl.fmap == "favor"
    halves = 2 if (wl.r if favor else wl.d_k) == 128 and wl.d_v == 128 else 1
    core = count - (4 if favor else 0)
    if not wl.causal or core % halves:
        return []
    per = core // halves
    one = {6: ["segment_state", "segment_scan", "bwd_pass_a", "bwd_rstate", "segment_scan_reverse", "bwd_pass_b"],
           2: ["bwd_pass_a", "bwd_pass_b"]}.get(per)
    if one is None:
        return []
    names = one if halves == 1 else [f"{k}_h{h}" for h in range(2) for k in one]
    if favor:
        names = ["favor_features_q", "favor_features_k"] + names + ["favor_vjp_q", "favor_vjp_k"]
    return names


def bench_backward(wl, steps, warmup):
    """la_backward on workload wl (causal; elu+1, FAVOR+ or identity features): one step is
    one full backward pass (with a gate input it includes dg, and dgv for the outer-product
    gate; with FAVOR+ the feature materialisation and the pass back through the map)."""
    import kernelized_sequence_mixing_amd as ksm
    from workloads import incoming_gradient
    inp = make_inputs(wl, seed=0)
    inp["dO"] = incoming_gradient((wl.B, wl.H, wl.n, wl.d_v), 1, dtype=wl.dtype)
    nb_tok, fl_tok = backward_algorithmic_per_token(wl)
    per_set = wl.head_tokens * nb_tok
    sets = _device_sets(inp, ["Q", "K", "V", "dO", "gamma", "g", "gv", "omega"], per_set)
    gate_of = {"none": lambda s: None, "decay": lambda s: ("decay", s["gamma"]),
               "gla": lambda s: ("gla", s["g"], wl.tau), "sel": lambda s: ("sel", s["g"], wl.tau),
               "outer": lambda s: ("outer", s["g"], s["gv"], wl.tau)}[wl.gate]
    grads = [(torch.empty_like(s["Q"]), torch.empty_like(s["K"]), torch.empty_like(s["V"])) +
             ((torch.empty_like(s["g"]),) if wl.gate in ("gla", "sel", "outer") else ()) +
             ((torch.empty_like(s["gv"]),) if wl.gate == "outer" else ()) for s in sets]
    stream = torch.cuda.current_stream()
    calls = [ksm.PreparedBackward(s["Q"], s["K"], s["V"], s["dO"], fmap=wl.fmap, omega=s.get("omega"),
                                  gate=gate_of(s), eps=wl.eps, grads=grads[i], stream=stream, causal=wl.causal)
             for i, s in enumerate(sets)]

    def step(i):
        calls[i]()

    ms, med = time_steps(step, len(sets), steps, warmup, stream)
    order = iter(range(10 ** 9))
    times = ksm.launch_times(lambda: calls[next(order) % len(calls)](), min(steps, 20), stream, max_launches=24)
    gbs = per_set / (ms * 1e-3) / 1e9
    tfl = wl.head_tokens * fl_tok / (ms * 1e-3) / 1e12
    return {"workload": wl.name + "_backward", "ms_per_step": round(ms, 5), "median_ms": round(med, 5),
            "value": wl.head_tokens / (ms * 1e-3), "unit": "head-tokens/s", "input_sets_rotated": len(sets),
            "kernels": kernel_table(times, backward_kernel_names(wl, len(times[0]))),
            "hbm_alg_GBs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "mfma_alg_TFLOPs": round(tfl, 2), "mfma_frac": round(tfl / BF16_PEAK_TFLOPS, 4),
            "alg_bytes_per_token": nb_tok, "alg_flops_per_token": fl_tok,
            "shape": {"B": wl.B, "H": wl.H, "n": wl.n, "d_k": wl.d_k, "d_v": wl.d_v, "gate": wl.gate,
                      "fmap": wl.fmap}}


def _host_info():
    cpu = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        cfg = np.show_config(mode="dicts")
        b = cfg.get("Build Dependencies", {}).get("blas", {})
        blas = f"{b.get('name', '?')} {b.get('version', '')}".strip()
    except Exception:  # noqa: BLE001 - the vendor string is informational only
        pass
    return cpu, blas


def cpu_baseline(wl, heads=32, block=64, max_threads=16):
    """The fp64 oracle's blocked form (oracle.causal_blocked, numpy) on the
    host: a bounded sample of `heads` whole heads of the workload (full
    sequence length), one head per worker thread, every thread running its
    BLAS single-threaded, so that all the host cores given to the process work
    at once. 64-token blocks: with a per-feature gate the block's decay tensor
    grows as block^2 r, and 64 is the fastest block on the host."""
    import oracle as orc
    from concurrent.futures import ThreadPoolExecutor
    from workloads import to_f64
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover - installed in this image
        threadpool_limits = None
    cores = len(os.sched_getaffinity(0))
    threads = max(1, min(cores, max_threads, heads))
    inp = make_inputs(wl, seed=0)
    sel = [(i // wl.H, i % wl.H) for i in range(min(heads, wl.B * wl.H))]
    gate = {"none": lambda b, h: None, "gla": lambda b, h: ("gla", to_f64(inp["g"][b:b + 1, h:h + 1]), wl.tau),
            "decay": lambda b, h: ("decay", to_f64(inp["gamma"][h:h + 1]))}[wl.gate]
    args = [(to_f64(inp["Q"][b:b + 1, h:h + 1]), to_f64(inp["K"][b:b + 1, h:h + 1]),
             to_f64(inp["V"][b:b + 1, h:h + 1]), gate(b, h)) for b, h in sel]

    def one(a):
        return orc.causal_blocked(a[0], a[1], a[2], wl.fmap, None, a[3], eps=wl.eps, block=block)[0].shape

    import contextlib
    with (threadpool_limits(limits=1) if threadpool_limits else contextlib.nullcontext()):
        r0 = resource.getrusage(resource.RUSAGE_SELF)
        t0 = time.perf_counter()
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, args))
        dt = time.perf_counter() - t0
        r1 = resource.getrusage(resource.RUSAGE_SELF)
    cpu_s = (r1.ru_utime - r0.ru_utime) + (r1.ru_stime - r0.ru_stime)
    model, blas = _host_info()
    toks = len(sel) * wl.n
    return {"value": toks / dt, "unit": "head-tokens/s", "cores": threads, "kind": "oracle", "seconds": round(dt, 2),
            "cpu_seconds": round(cpu_s, 1),
            "sample": f"{wl.name}: {len(sel)} of the {wl.B * wl.H} heads, each the whole n={wl.n} sequence "
                      f"(d_k=d_v={wl.d_k}, gate {wl.gate}), fp64 numpy blocked form in {block}-token blocks, "
                      f"{threads} worker threads with single-threaded BLAS",
            "host_cores_available": cores, "cpu_model": model, "blas": blas}


CROSSOVER_N = (1024, 2048, 4096, 8192, 16384, 32768)


def bench_softmax(n, steps, warmup, B=4, H=16, d=64):
    """The softmax-attention baseline (la_softmax_attention, causal, bf16) at
    B4 H16 d64 and sequence length n: the quadratic form linear attention
    replaces. Flops per head: 2 n^2 d (the scores and the weighted values, each
    2 n^2 d / 2 over the causal triangle)."""
    import kernelized_sequence_mixing_amd as ksm
    wl = WORKLOADS["causal_elu1"].resized(name=f"softmax_n{n}", B=B, H=H, n=n, qk_scale=1.0, v_scale=1.0)
    inp = make_inputs(wl, seed=0)
    per_set = B * H * n * 4 * d * 2
    sets = _device_sets(inp, ["Q", "K", "V"], per_set)
    outs = [torch.empty_like(s["V"]) for s in sets]
    stream = torch.cuda.current_stream()
    calls = [ksm.PreparedSoftmax(s["Q"], s["K"], s["V"], causal=True, out=outs[i], stream=stream)
             for i, s in enumerate(sets)]
    ms, med = time_steps(lambda i: calls[i](), len(sets), steps, warmup, stream)
    flops = 2.0 * n * n * d * B * H
    tfl = flops / (ms * 1e-3) / 1e12
    return {"workload": f"softmax_causal_n{n}", "ms_per_step": round(ms, 5), "median_ms": round(med, 5),
            "value": B * H * n / (ms * 1e-3), "unit": "head-tokens/s", "input_sets_rotated": len(sets),
            "mfma_alg_TFLOPs": round(tfl, 2), "mfma_frac": round(tfl / BF16_PEAK_TFLOPS, 4),
            "score_matrix_fp16_bytes_per_head": n * n * 2,
            "shape": {"B": B, "H": H, "n": n, "d": d, "causal": True}}


def bench_crossover(steps, warmup):
    """Softmax attention and causal elu+1 linear attention at the same B4 H16
    d64 for each n of CROSSOVER_N: head-tokens/s of both, and the ratio."""
    rows = []
    for n in CROSSOVER_N:
        st = max(3, steps // (n // 4096 + 1)) if n > 4096 else steps
        sm = bench_softmax(n, st, min(warmup, 2), d=64)
        lin = bench_forward(WORKLOADS["causal_elu1"].resized(name=f"causal_elu1_n{n}", n=n), st, min(warmup, 2))
        rows.append({"n": n, "softmax_head_tokens_per_s": sm["value"], "softmax_ms": sm["ms_per_step"],
                     "softmax_mfma_frac": sm["mfma_frac"], "linear_head_tokens_per_s": lin["value"],
                     "linear_ms": lin["ms_per_step"], "linear_over_softmax": round(lin["value"] / sm["value"], 3)})
        print(f"crossover n={n}: softmax {sm['ms_per_step']:.4f} ms ({sm['mfma_frac']:.3f} of MFMA peak), "
              f"linear {lin['ms_per_step']:.4f} ms", file=sys.stderr, flush=True)
    return {"workload": "crossover_softmax_vs_linear_B4_H16_d64", "rows": rows}


def run_only(name, steps, warmup):
    """One workload's record alone (for per-workload profiles)."""
    if name in WORKLOADS and not WORKLOADS[name].decode:
        return bench_forward(WORKLOADS[name], steps, warmup)
    if name == "gla_decode":
        return bench_decode(WORKLOADS[name], steps, warmup)
    if name == "serve_prefill":
        return bench_serve_prefill(steps, warmup)
    if name in ("serve_decode_m1", "serve_decode_m4"):
        return bench_serve_decode(WORKLOADS["gla_decode"], int(name[-1]), steps, warmup)
    if name.startswith("softmax_n"):
        return bench_softmax(int(name[len("softmax_n"):]), steps, warmup)
    if name == "crossover":
        return bench_crossover(steps, warmup)
    if name.endswith("_backward") and name[:-len("_backward")] in BACKWARD_WORKLOADS:
        return bench_backward(BACKWARD_WORKLOADS[name[:-len("_backward")]], steps, warmup)
    raise SystemExit(f"unknown workload {name!r}")


# the backward lines: the GLA, outer-product-gate and RetNet workloads at their own shapes (128 x 128
# states, two value-column halves), the ungated elu+1 shape, the GLA sequence shape at d_k = d_v = 64,
# the state-space form under both selective gates, non-causal, FAVOR+ at the causal FAVOR+ shape with
# r = 128 (the widest feature count the backward builds)
BACKWARD_WORKLOADS = {
    "gla_gate": WORKLOADS["gla_gate"],
    "outer_gate": WORKLOADS["outer_gate"],
    "retnet_decay": WORKLOADS["retnet_decay"],
    "causal_elu1": WORKLOADS["causal_elu1"],
    "gla_gate_d64": WORKLOADS["gla_gate"].resized(name="gla_gate_d64", d_k=64, d_v=64, r=64, qk_scale=64 ** -0.5,
                                                  v_scale=64 ** -0.5),
    "ssm_selective": WORKLOADS["ssm_selective"],
    "ssm_scalar": WORKLOADS["ssm_scalar"],
    "noncausal_elu1_f32": WORKLOADS["noncausal_elu1_f32"],
    "favor_r128": WORKLOADS["favor_causal"].resized(name="favor_r128", r=128),
}


def roofline(wl, res):
    """The dominant kernel of a forward step against the HBM roofline:
    algorithmic bytes of the whole step (every head-token's q, k, v, gate
    inputs read once and o written once, all of them by the output pass) over
    that kernel's average launch time from the per-launch events."""
    nb_tok, _ = algorithmic_per_token(wl)
    dom = max(res["kernels"], key=lambda k: k["avg_ms"])
    alg = wl.head_tokens * nb_tok
    gbs = alg / (dom["avg_ms"] * 1e-3) / 1e9
    tr = measured_traffic(wl.name, dom["name"])
    return {"bound": "hbm", "kernel": dom["name"], "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": tr, "alg_bytes_per_launch": alg,
            "launch_ms": dom["avg_ms"],
            "step": {"achieved": res["hbm_alg_GBs"], "frac": res["hbm_frac"], "ms": res["ms_per_step"]}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-extra", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default=None, help="run one workload and print its record alone")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (scales the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a visible MI355X", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.copy_calibration:
        nbytes = 1 << 30
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": True, "bytes_read_per_copy": nbytes, "bytes_written_per_copy": nbytes,
                          "copies": 5}), flush=True)
        return
    from kernelized_sequence_mixing_amd import _native
    _native.lib()  # fail loudly if the HIP library is missing
    if args.only:
        print(json.dumps(run_only(args.only, args.steps, args.warmup)), flush=True)
        return

    wl = WORKLOADS[HEADLINE]
    head = bench_forward(wl, args.steps, args.warmup)
    print(f"headline {wl.name}: {head['ms_per_step']:.4f} ms/step, kernels {head['kernels']}", file=sys.stderr,
          flush=True)
    line = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1)*d^-0.5 inputs, N(0,1) gate inputs, rotated copies in HBM)",
        "config": {"workload": "GLA-gated causal elu+1 linear attention forward, B=2 H=16 n=16384 d_k=d_v=128, "
                               "bf16 in/out, fp32 state, chunk 64, tau 16", "B": wl.B, "H": wl.H, "n": wl.n,
                   "d_k": wl.d_k, "d_v": wl.d_v, "feature_map": "elu+1", "gate": "gla", "chunk": CHUNK},
        "kernels": head["kernels"],
        "roofline": roofline(wl, head),
        "mfma": {"alg_TFLOPs": head["mfma_alg_TFLOPs"], "peak_TFLOPs": BF16_PEAK_TFLOPS,
                 "alg_frac": head["mfma_frac"],
                 "counter": measured_mfma(wl.name, max(head["kernels"], key=lambda k: k["avg_ms"])["name"]),
                 "note": "alg_*: algorithmic flops over the step time; counter: the dominant kernel's rocprofv3 "
                         "summary in profiles/ (null if taken on other kernel sources)"},
        "context": {"softmax_score_matrix_n16384_fp16_bytes": 16384 * 16384 * 2},
    }
    if not args.no_extra:
        extra = []
        for name in ("noncausal_elu1_f32", "causal_elu1", "retnet_decay", "outer_gate", "ssm_selective", "ssm_scalar",
                     "favor_causal"):
            r = bench_forward(WORKLOADS[name], args.steps, args.warmup)
            if WORKLOADS[name].causal:
                r["roofline"] = roofline(WORKLOADS[name], r)
            extra.append(r)
            print(f"{name}: {r['ms_per_step']:.4f} ms/step", file=sys.stderr, flush=True)
        extra.append(bench_decode(WORKLOADS["gla_decode"], args.steps, args.warmup))
        extra.append(bench_serve_prefill(args.steps, args.warmup))
        for m in (1, 4):
            extra.append(bench_serve_decode(WORKLOADS["gla_decode"], m, args.steps, args.warmup))
        for bw in BACKWARD_WORKLOADS.values():
            extra.append(bench_backward(bw, args.steps, args.warmup))
            print(f"{bw.name} backward: {extra[-1]['ms_per_step']:.4f} ms/step", file=sys.stderr, flush=True)
        extra.append(bench_crossover(args.steps, args.warmup))
        line["extra"] = extra
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
