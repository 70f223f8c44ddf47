"""Benchmark: causal kernelized linear attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu-baseline]

A step is one full forward pass of the hot path (feature map, segment states,
segment chaining, chunked outputs) over one batch of the headline workload:
causal elu+1, B=4 H=16 n=4096 d_k=d_v=64, bf16 inputs, fp32 state, 64-token
chunks. Inputs are seeded synthetic tensors already resident in HBM; several
copies at different addresses are rotated so that consecutive steps do not
find their inputs in the 256 MB last-level (MALL) cache. Timing uses HIP events
on the stream the library launches on. Rank 0 prints one JSON line.

The same line carries, under "extra", the other workloads (non-causal fp32,
RetNet decay, GLA gate, FAVOR+, the GLA decode step, and the backward pass on
the headline shape), and the fp64 CPU oracle timed on the host on a bounded
sample of the headline workload.
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


def measured_traffic(workload):
    """HBM bytes per step from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_digest") != source_digest():
        return None
    return t.get("hbm_bytes_per_step")


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
    tok_s = wl.head_tokens / (ms * 1e-3)
    res = {"workload": wl.name, "ms_per_step": round(ms, 5), "median_ms": round(med, 5),
           "value": tok_s, "unit": "head-tokens/s", "input_sets_rotated": len(sets)}
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
    write dg, r per token each; the selective gate: one of each per token). Flops (chunk C, masked upper triangle excluded): the scores, the
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
    half = (CHUNK + 1) / 2
    flops = half * 2 * wl.r * 3 + half * 2 * wl.d_v * 3 + 6 * 2 * wl.r * wl.d_v
    if not wl.causal:  # the non-causal form: S, G and the per-token products, no scores
        flops = 6 * 2 * wl.r * wl.d_v
    return nbytes, flops


def bench_backward(wl, steps, warmup):
    """la_backward on workload wl (causal, elu+1 or identity features): one step is one
    full backward pass (with a gate input it includes dg)."""
    import kernelized_sequence_mixing_amd as ksm
    from workloads import incoming_gradient
    inp = make_inputs(wl, seed=0)
    inp["dO"] = incoming_gradient((wl.B, wl.H, wl.n, wl.d_v), 1, dtype=wl.dtype)
    nb_tok, fl_tok = backward_algorithmic_per_token(wl)
    per_set = wl.head_tokens * nb_tok
    sets = _device_sets(inp, ["Q", "K", "V", "dO", "gamma", "g"], per_set)
    gate_of = {"none": lambda s: None, "decay": lambda s: ("decay", s["gamma"]),
               "gla": lambda s: ("gla", s["g"], wl.tau), "sel": lambda s: ("sel", s["g"], wl.tau)}[wl.gate]
    grads = [(torch.empty_like(s["Q"]), torch.empty_like(s["K"]), torch.empty_like(s["V"])) +
             ((torch.empty_like(s["g"]),) if wl.gate in ("gla", "sel") else ()) for s in sets]
    stream = torch.cuda.current_stream()
    calls = [ksm.PreparedBackward(s["Q"], s["K"], s["V"], s["dO"], fmap=wl.fmap, gate=gate_of(s), eps=wl.eps,
                                  grads=grads[i], stream=stream, causal=wl.causal) for i, s in enumerate(sets)]

    def step(i):
        calls[i]()

    ms, med = time_steps(step, len(sets), steps, warmup, stream)
    gbs = per_set / (ms * 1e-3) / 1e9
    tfl = wl.head_tokens * fl_tok / (ms * 1e-3) / 1e12
    return {"workload": wl.name + "_backward", "ms_per_step": round(ms, 5), "median_ms": round(med, 5),
            "value": wl.head_tokens / (ms * 1e-3), "unit": "head-tokens/s", "input_sets_rotated": len(sets),
            "hbm_alg_GBs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "mfma_alg_TFLOPs": round(tfl, 2), "mfma_frac": round(tfl / BF16_PEAK_TFLOPS, 4),
            "alg_bytes_per_token": nb_tok, "alg_flops_per_token": fl_tok,
            "shape": {"B": wl.B, "H": wl.H, "n": wl.n, "d_k": wl.d_k, "d_v": wl.d_v, "gate": wl.gate,
                      "fmap": wl.fmap}}


def cpu_baseline(wl, min_seconds=10.0):
    """The fp64 oracle (recurrent form, numpy) on the host: whole passes over
    all heads of the headline workload, repeated until about `min_seconds` of
    CPU work has been timed."""
    import oracle as orc
    from workloads import to_f64
    inp = make_inputs(wl, seed=0)
    Q, K, V = (to_f64(inp[k]) for k in ("Q", "K", "V"))
    r0 = resource.getrusage(resource.RUSAGE_SELF)
    t0 = time.perf_counter()
    passes = 0
    while True:
        orc.causal_recurrent(Q, K, V, wl.fmap, None, None, eps=wl.eps)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or passes >= 20:
            break
    r1 = resource.getrusage(resource.RUSAGE_SELF)
    cpu = (r1.ru_utime - r0.ru_utime) + (r1.ru_stime - r0.ru_stime)
    return {"value": passes * wl.head_tokens / dt, "unit": "head-tokens/s", "cores": max(1, round(cpu / dt)),
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"{wl.name}: {passes} full passes over all B*H={wl.B * wl.H} heads x n={wl.n} tokens, "
                      "fp64 numpy recurrent form",
            "host": platform.processor() or platform.machine()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-extra", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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

    wl = WORKLOADS[HEADLINE]
    head = bench_forward(wl, args.steps, args.warmup)
    traffic = measured_traffic(wl.name)
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
        "data": "synthetic (seeded N(0,1)*d^-0.5 inputs, rotated copies in HBM)",
        "config": {"workload": "causal elu+1 linear attention forward, B=4 H=16 n=4096 d_k=d_v=64, bf16 in/out, "
                               "fp32 state, chunk 64", "B": wl.B, "H": wl.H, "n": wl.n, "d_k": wl.d_k,
                   "d_v": wl.d_v, "feature_map": "elu+1", "gate": "none", "chunk": CHUNK},
        "roofline": {"bound": "hbm", "kernel": "la_forward step (segment-state pass + scan + chunked output pass)",
                     "achieved": head["hbm_alg_GBs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": head["hbm_frac"], "traffic": traffic,
                     "alg_bytes_per_launch": wl.head_tokens * head["alg_bytes_per_token"]},
        "mfma": {"achieved_TFLOPs": head["mfma_alg_TFLOPs"], "peak_TFLOPs": BF16_PEAK_TFLOPS,
                 "frac": head["mfma_frac"]},
        "context": {"softmax_score_matrix_n16384_fp16_bytes": 16384 * 16384 * 2},
    }
    if not args.no_extra:
        extra = []
        for name in ("noncausal_elu1_f32", "retnet_decay", "gla_gate", "outer_gate", "ssm_selective", "ssm_scalar",
                     "favor_causal"):
            extra.append(bench_forward(WORKLOADS[name], args.steps, args.warmup))
        extra.append(bench_decode(WORKLOADS["gla_decode"], args.steps, args.warmup))
        extra.append(bench_serve_prefill(args.steps, args.warmup))
        for m in (1, 4):
            extra.append(bench_serve_decode(WORKLOADS["gla_decode"], m, args.steps, args.warmup))
        extra.append(bench_backward(WORKLOADS["causal_elu1"], args.steps, args.warmup))
        # the GLA workload's sequence shape at d_k = d_v = 64 (no backward build for 128 x 128 states)
        extra.append(bench_backward(WORKLOADS["gla_gate"].resized(name="gla_gate_d64", d_k=64, d_v=64, r=64,
                                                                  qk_scale=64 ** -0.5, v_scale=64 ** -0.5),
                                    args.steps, args.warmup))
        for name in ("ssm_selective", "ssm_scalar"):  # the state-space form under both selective gates
            extra.append(bench_backward(WORKLOADS[name], args.steps, args.warmup))
        extra.append(bench_backward(WORKLOADS["noncausal_elu1_f32"], args.steps, args.warmup))
        line["extra"] = extra
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
