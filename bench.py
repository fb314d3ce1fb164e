#!/usr/bin/env python3
"""Throughput of one tensor-parallel rank's pre-LN layer shard, forward +
backward, on one MI355X, through the C ABI of libtplayer.so.

A step is one tp_layer_fwd(TP_ALL) + tp_layer_bwd(TP_ALL) over one
micro-batch of seeded synthetic input already resident in HBM. The metric is
algorithmic TFLOP/s (GEMMs 2MNK, attention 4*dh*H_l per allowed query-key
pair, backward = 2x forward; no recomputation, masked work, LayerNorm or
elementwise work counted) and its fraction of the bf16 dense MFMA peak.

With `--mode decode` a step is instead one decode step of the same shard
(tp_layer_decode, TP_ALL): one new token for each of the micro-batch's
sequences against a KV cache shard of `--cache-len` rows; the metric is
generated tokens per second and the roofline is HBM bandwidth (weights and
cache rows read once per step).

Prints ONE JSON line. `--gpus N` with N > 1 exits: this build runs one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK = {"bf16": (2500.0, "TFLOP/s"), "f32": (157.3, "TFLOP/s")}  # MI355X dense MFMA / fp32 vector
HBM_PEAK_GBS = 8000.0
METRIC = "TFLOP/s per GPU, fwd+bwd of one TP-rank layer shard; % of bf16 MFMA peak"


def algorithmic_flops(d, valid_len):
    n = d.tokens
    gemm = 2 * n * (d.hidden * 3 * d.hidden_local + d.hidden_local * d.hidden
                    + d.hidden * d.ffn_local + d.ffn_local * d.hidden)
    if d.mask == "causal":
        pairs = d.batch * d.seq * (d.seq + 1) // 2
    else:
        pairs = d.seq * int(sum(int(v) for v in valid_len))
    return 3 * (gemm + 4 * d.head_dim * d.heads_local * pairs)


def _blas_info():
    """Vendor, version and thread count of the BLAS NumPy runs the oracle on."""
    try:
        import numpy  # noqa: F401  (loads the BLAS that threadpoolctl inspects)
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                return {"blas": f"{i.get('internal_api')} {i.get('version')}",
                        "threads": int(i.get("num_threads", 1))}
    except Exception:
        pass
    return {"blas": "unknown", "threads": os.cpu_count() or 1}


def _physical_cores():
    """Physical cores of the host (distinct (package, core) pairs), or None."""
    try:
        seen = set()
        base = "/sys/devices/system/cpu"
        for c in os.listdir(base):
            if not (c.startswith("cpu") and c[3:].isdigit()):
                continue
            topo = os.path.join(base, c, "topology")
            with open(os.path.join(topo, "physical_package_id")) as f:
                pkg = f.read().strip()
            with open(os.path.join(topo, "core_id")) as f:
                core = f.read().strip()
            seen.add((pkg, core))
        return len(seen) or None
    except Exception:
        return None


def cpu_baseline(w, tokens, min_seconds, params=None):
    """The fp64 oracle timed on the host on a bounded sample of the shard:
    the same layer shard (same hidden, heads, FFN, t, rank, weights) over
    `tokens` tokens -- whole sequences when the micro-batch has several, else
    the first `tokens` positions of the sequence -- forward + backward, repeated
    until `min_seconds` of CPU work have run. The rate is the sample's
    algorithmic FLOPs over the time, the same count the GPU figure uses."""
    from oracle import layer as OL
    from tensor_model_transformer_amd.synth import layer_inputs, rank_params

    d = w.dims
    if d.batch > 1:
        seqs = max(1, min(d.batch, tokens // d.seq))
        dims = d.__class__(seqs, d.seq, d.hidden, d.heads, d.ffn, d.t, d.dtype, d.mask)
        what = f"{seqs} of {d.batch} sequences"
    else:
        s = max(1, min(d.seq, tokens))
        dims = d.__class__(1, s, d.hidden, d.heads, d.ffn, d.t, d.dtype, d.mask)
        what = f"the first {s} of {d.seq} positions"
    ws = w.with_(dims=dims)
    if params is None:
        params = rank_params(ws)
    x, dout, vl = layer_inputs(ws)
    info = _blas_info()
    reps, dt = 0, 0.0
    while reps == 0 or dt < min_seconds:
        t0 = time.perf_counter()
        OL.layer_local(params, x, dout, ws.dims, vl)
        dt += time.perf_counter() - t0
        reps += 1
    f = algorithmic_flops(ws.dims, vl)
    return {"value": reps * f / dt / 1e12, "unit": "TFLOP/s", "cores": info["threads"],
            "kind": "oracle", "seconds": dt, "blas": info["blas"],
            "physical_cores": _physical_cores(), "logical_cpus": os.cpu_count(),
            "sample": f"{what} of the {w.name} shard ({ws.dims.tokens} tokens; same weights "
                      f"and widths), fp64 NumPy oracle, LOCAL mode, fwd+bwd, "
                      f"{f / 1e9:.1f} GFLOP, run {reps}x"}


class SclkSampler:
    """Samples the GPU's graphics clock (SCLK) from sysfs during a timed
    region: the current level of pp_dpm_sclk of the device's PCI function,
    read every few milliseconds on a host thread (no GPU call, no process)."""

    def __init__(self, device_index=0, period_s=0.005):
        self.path, self.err = self._find(device_index), None
        self.period = period_s
        self.samples = []
        self._stop = None
        self._thread = None

    @staticmethod
    def _find(idx):
        import glob
        import torch
        try:
            p = torch.cuda.get_device_properties(idx)
            bdf = "%04x:%02x:%02x.0" % (int(getattr(p, "pci_domain_id")),
                                        int(getattr(p, "pci_bus_id")),
                                        int(getattr(p, "pci_device_id")))
            cand = f"/sys/bus/pci/devices/{bdf}/pp_dpm_sclk"
            if os.path.exists(cand):
                return cand
        except Exception:
            pass
        found = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        return found[0] if len(found) == 1 else None

    def _read(self):
        with open(self.path) as f:
            for line in f:
                if "*" in line:
                    tok = line.split(":", 1)[1].strip().split()[0].lower()
                    return float(tok.replace("mhz", ""))
        return None

    def start(self):
        import threading
        if not self.path:
            self.err = "no pp_dpm_sclk found for the device"
            return self
        self._stop = threading.Event()

        def run():
            while not self._stop.is_set():
                try:
                    v = self._read()
                    if v:
                        self.samples.append(v)
                except Exception as e:  # noqa: BLE001
                    self.err = str(e)
                    return
                time.sleep(self.period)

        self._thread = threading.Thread(target=run, daemon=True)
        self._thread.start()
        return self

    def stop(self):
        if self._thread:
            self._stop.set()
            self._thread.join()
        if not self.samples:
            return {"mhz_median": None, "samples": 0, "source": self.path,
                    "note": self.err or "no samples"}
        v = sorted(self.samples)
        return {"mhz_median": v[len(v) // 2], "mhz_min": v[0], "mhz_max": v[-1],
                "samples": len(v), "source": self.path}


def source_digest(paths):
    """sha256 over the given kernel sources, in order; ties a stored counter
    reading to the code it was taken from."""
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


# Kernel sources whose counter readings a traffic summary holds, per kernel class.
TRAFFIC_SOURCES = {"gemm": ["tensor_model_transformer_amd/csrc/gemm.hip",
                            "tensor_model_transformer_amd/csrc/common.hpp"]}


def stored_traffic(kclass, workload):
    """HBM bytes per launch of `kclass` on `workload`, from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary, already scaled by the copy-kernel
    calibration; None when there is no summary or the kernel source changed
    since the counters were read."""
    path = os.path.join(ROOT, "profiles", f"{kclass}_traffic_{workload}.md")
    if kclass not in TRAFFIC_SOURCES or not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].split(": ", 1)
                kv[k.strip("` ")] = v.strip().strip("`")
    if kv.get("source_sha256") != source_digest(TRAFFIC_SOURCES[kclass]):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_probe(nbytes, reps):
    """A plain copy of known size through the library's own exchange kernel
    (one fp32 part in, fp32 out): the calibration run for the FETCH_SIZE and
    WRITE_SIZE counters."""
    import torch
    from tensor_model_transformer_amd import binding as B
    from tensor_model_transformer_amd.shard import exchange_sum
    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(reps):
        exchange_sum(dst, [src], stream)
    torch.cuda.synchronize()
    assert bool((dst == 1).all()), "copy probe produced wrong values"
    print(json.dumps({"copy_probe_bytes_read": 4 * n, "copy_probe_bytes_written": 4 * n,
                      "reps": reps, "kernel": "tp_exchange_sum(1 part, f32)",
                      "dtype_code": B.TP_DTYPE_F32}))


DECODE_METRIC = ("decode tokens/s per GPU, one TP-rank layer shard, one new token per sequence "
                 "against its KV cache shard")


def decode_bytes(d, positions, split_scores):
    """Algorithmic HBM bytes of one decode step of one rank: every weight and
    bias read once, cache rows 0..pos read once per sequence (K, V, and the K
    residuals with split scores), the new K and V rows written, the token rows
    read and the output written once. The [B, h] intermediates between the
    kernels are not counted."""
    e = 2 if d.dtype == "bf16" else 4
    h, hl, fl, B = d.hidden, d.hidden_local, d.ffn_local, d.batch
    weights = (h * 3 * hl + hl * h + h * fl + fl * h) * e + (6 * h + 3 * hl + fl) * e
    keys = sum(int(p) + 1 for p in positions)
    per_key = hl * e * (3 if split_scores else 2)
    return weights + keys * per_key + 2 * B * hl * e + 2 * B * h * e


def cpu_decode_baseline(w, cache_len, min_seconds):
    """The fp64 decode oracle timed on the host: the same decode step (all
    sequences, full cache), repeated until `min_seconds` have run."""
    from oracle import decode as OD
    from tensor_model_transformer_amd.synth import decode_inputs, rank_caches, rank_params
    d = w.dims
    params = rank_params(w)
    x, pos = decode_inputs(w, cache_len, "full")
    kc, vc = rank_caches(w, w.rank, cache_len)
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    reps, dt = 0, 0.0
    while reps == 0 or dt < min_seconds:
        t0 = time.perf_counter()
        OD.decode_step(params, x, kc, vc, pos, d.heads_local)
        dt += time.perf_counter() - t0
        reps += 1
    return {"value": reps * d.batch / dt, "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle", "seconds": dt,
            "sample": f"the whole decode step ({d.batch} sequences at position {cache_len - 1}) "
                      f"of the {w.name} shard, fp64 NumPy oracle, run {reps}x"}


def bench_decode(args):
    import torch
    from tensor_model_transformer_amd import binding as B
    from tensor_model_transformer_amd.shard import Shard, _check
    from tensor_model_transformer_amd.synth import WORKLOADS, decode_inputs, rank_caches, rank_params

    w = WORKLOADS[args.workload]
    d = w.dims
    if d.mask != "causal":
        print(f"bench.py: {w.name} is a bidirectional (padding-mask) layer; decode needs a causal "
              "one", file=sys.stderr)
        sys.exit(2)
    L = args.cache_len or d.seq
    sh = Shard(d, w.rank)
    p = sh.upload_params(rank_params(w))
    x, pos = decode_inputs(w, L, "full")
    kc, vc = rank_caches(w, w.rank, L)
    xd = torch.from_numpy(x).to(sh.device).to(sh.dtype)
    kd, vd = sh.upload_cache(kc), sh.upload_cache(vc)
    del kc, vc
    split = sh.split_scores
    klo = torch.zeros_like(kd) if split else None
    posd = torch.from_numpy(pos).to(sh.device)
    out = torch.empty(d.batch, d.hidden, dtype=sh.dtype, device=sh.device)
    sh.decode_workspace()
    stream = torch.cuda.Stream(device=sh.device)

    def step():
        _check("tp_layer_decode", sh.decode(p, out, x=xd, k_cache=kd, v_cache=vd,
                                            k_cache_lo=klo, positions=posd))

    def timed(fn, n):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(n):
            fn()
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / n

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
        t0 = time.perf_counter()
        ms_per_step = timed(step, args.steps)
        wall = time.perf_counter() - t0
        # the same step captured once in a HIP graph and replayed (reported
        # beside the direct calls, which are faster on this stack)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            step()
        for _ in range(args.warmup):
            graph.replay()
        graph_ms = timed(graph.replay, args.steps)
    value = d.batch / (ms_per_step * 1e-3)
    nbytes = decode_bytes(d, pos, split)
    print(f"[bench] decode {w.name} B={d.batch} L={L}: {ms_per_step * 1e3:.1f} us/step, "
          f"{graph_ms * 1e3:.1f} us/step graph replay, {value:.0f} tokens/s, "
          f"{nbytes / ms_per_step / 1e6:.0f} GB/s (wall {wall:.2f} s)", file=sys.stderr, flush=True)

    # per-kernel-class event timing over eager steps
    _check("tp_layer_profile", B.tp_layer_profile(sh.handle, 1))
    with torch.cuda.stream(stream):
        for _ in range(args.steps):
            step()
    torch.cuda.synchronize()
    breakdown = {}
    for k in B.KCLASSES:
        rc, n, kms, kfl, kby = B.tp_layer_profile_read(sh.handle, k)
        _check("tp_layer_profile_read", rc)
        if n:
            breakdown[k] = {"launches_per_step": n / args.steps, "ms_per_step": kms / args.steps,
                            "gbyte_per_step": kby / args.steps / 1e9}
    B.tp_layer_profile(sh.handle, 0)
    dom = max(breakdown, key=lambda k: breakdown[k]["ms_per_step"])
    bd = breakdown[dom]
    achieved = bd["gbyte_per_step"] / bd["ms_per_step"] * 1e3
    roof = {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": None,
            "algorithmic_bytes_per_launch": bd["gbyte_per_step"] * 1e9 / bd["launches_per_step"],
            "launches_per_step": bd["launches_per_step"],
            "avg_launch_ms": bd["ms_per_step"] / bd["launches_per_step"],
            "step_bytes": nbytes, "step_gbs": nbytes / ms_per_step / 1e6,
            "step_frac": nbytes / ms_per_step / 1e6 / HBM_PEAK_GBS}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_decode_baseline(w, L, args.cpu_min_seconds)
        print(f"[bench] cpu oracle: {cpu['value']:.1f} tokens/s on {cpu['cores']} threads",
              file=sys.stderr, flush=True)
    line = {
        "metric": DECODE_METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": d.dtype, "data": "synthetic (seeded N(0,1) tokens, N(0,0.02) weights, "
                                  "N(0, (0.02 sqrt h)^2) cache)",
        "config": {"workload": f"decode_{w.name}", "decode_batch": d.batch, "cache_len": L,
                   "positions": "all at cache_len - 1", "hidden": d.hidden, "heads": d.heads,
                   "ffn": d.ffn, "t": d.t, "rank": w.rank, "split_scores": split,
                   "launch": "direct C-ABI calls", "graph_replay_ms_per_step": graph_ms,
                   "decode_workspace_bytes": sh.dws_bytes},
        "roofline": roof, "cpu_baseline": cpu, "breakdown": breakdown,
    }
    print(json.dumps(line))
    del graph
    sh.close()


# The shard the headline is quoted on: the largest single-GPU configuration,
# the 1T GPT's rank 0 of 8 (b 1, s 2048, h 25600, 160 heads, FFN 102400). The
# other measured shards are reported beside it.
DEFAULT_WORKLOAD = "gpt_1t_t8"
OTHER_WORKLOADS = ("gpt_1p2b_t1", "gpt_8p3b_t8", "bert_3p9b_t4")


def timed_steps(step, steps, warmup, sclk=None):
    """Runs `warmup` untimed steps, then `steps` steps each bracketed by its
    own pair of HIP events on the launch stream (no host sync in between).
    Returns the per-step milliseconds, the whole bracket's milliseconds, the
    wall seconds and the clock samples."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    if sclk:
        sclk.start()
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(steps):
        step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    clock = sclk.stop() if sclk else None
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return per, ev[0].elapsed_time(ev[steps]), wall, clock


def _median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


def make_train_step(w, sp=False, recompute=False, params=None, overlap=0):
    """Uploads the workload and returns (step, shard, valid_len, cleanup)."""
    import torch
    from tensor_model_transformer_amd import binding as B
    from tensor_model_transformer_amd.shard import Shard, _check
    from tensor_model_transformer_amd.synth import layer_inputs, rank_params

    d = w.dims
    if params is None:
        params = rank_params(w)
    x, dout, vl = layer_inputs(w)
    sh = Shard(d, w.rank, recompute=B.TP_RECOMPUTE_FC1 if recompute else B.TP_RECOMPUTE_NONE,
               sequence_parallel=sp, overlap=overlap)
    p = sh.upload_params(params, vl if d.mask == "padding" else None)
    xd, doutd = sh.act(x), sh.act(dout)
    out, dx = sh.empty_act(), sh.empty_dx()
    grads = sh.zero_grads()

    def step():
        _check("tp_layer_fwd", sh.fwd(p, out, x=xd))
        _check("tp_layer_bwd", sh.bwd(p, grads, x=xd, dout=doutd, dx=dx))

    if sp:
        # One rank's sequence-parallel share: LayerNorms, biases and residuals on
        # its n/t rows, GEMMs and attention on all n rows. The gathered and
        # reduced tensors the collectives would deliver are stand-ins here
        # (their values do not change the work); the collectives themselves
        # are not part of one rank's kernels and are not timed.
        nc = d.tokens // d.t
        rows = slice(w.rank * nc, (w.rank + 1) * nc)
        act = torch.float16 if d.dtype == "bf16" else torch.float32
        gen = torch.Generator(device="cuda").manual_seed(7)
        g_a = torch.randn(d.tokens, d.hidden, generator=gen, device="cuda").to(act)
        g_c = torch.randn(d.tokens, d.hidden, generator=gen, device="cuda").to(act)
        g_dh = torch.randn(d.tokens, d.hidden, generator=gen, device="cuda").to(act)
        red = torch.randn(nc, d.hidden, generator=gen, device="cuda")
        part = sh.empty_act(fp32=True)
        x_r, dout_r, out_r, dx_r = xd[rows], doutd[rows], out[rows], dx[rows]

        def step():  # noqa: F811
            F, Bw = sh.fwd, sh.bwd
            _check("sp ln1", F(p, None, x=x_r, gathered=g_a, phase=B.TP_FWD_SP_LN1))
            _check("sp attn", F(p, part, gathered=g_a, phase=B.TP_FWD_SP_ATTN))
            _check("sp ln2", F(p, None, x=x_r, reduced=red, gathered=g_c, phase=B.TP_FWD_SP_LN2))
            _check("sp mlp", F(p, part, gathered=g_c, phase=B.TP_FWD_SP_MLP))
            _check("sp out", F(p, out_r, reduced=red, phase=B.TP_FWD_SP_OUT))
            _check("sp bwd mlp", Bw(p, grads, dout=dout_r, gathered_grad=doutd, gathered_act=g_c,
                                    partial=part, phase=B.TP_BWD_SP_MLP))
            _check("sp bwd ln2", Bw(p, grads, dc=red, dout=dout_r, gathered_grad=g_dh,
                                    phase=B.TP_BWD_SP_LN2))
            _check("sp bwd attn", Bw(p, grads, gathered_grad=g_dh, gathered_act=g_a, partial=part,
                                     phase=B.TP_BWD_SP_ATTN))
            _check("sp bwd ln1", Bw(p, grads, da=red, x=x_r, dx=dx_r, phase=B.TP_BWD_SP_LN1))

    def cleanup():
        sh.close()

    return step, sh, vl, cleanup


def step_stats(per, flops):
    med = _median(per)
    return {"ms_per_step": med, "ms_min": min(per), "ms_max": max(per),
            "ms_mean": sum(per) / len(per), "value": flops / (med * 1e-3) / 1e12,
            "pct_of_peak": 100.0 * flops / (med * 1e-3) / 1e12 / PEAK["bf16"][0]}


def bench_train(args):
    import torch
    from tensor_model_transformer_amd import binding as B
    from tensor_model_transformer_amd.shard import _check
    from tensor_model_transformer_amd.synth import WORKLOADS, rank_params

    w = WORKLOADS[args.workload]
    d = w.dims
    sp = args.layout == "sp"
    params = rank_params(w)
    overlap = {"auto": B.TP_OVERLAP_AUTO, "off": B.TP_OVERLAP_OFF,
               "on": B.TP_OVERLAP_ON}[args.overlap]
    step, sh, vl, cleanup = make_train_step(w, sp, args.recompute, params, overlap)
    flops = algorithmic_flops(d, vl)
    sclk = None if args.no_sclk else SclkSampler()
    per, bracket_ms, wall, clock = timed_steps(step, args.steps, args.warmup, sclk)
    st = step_stats(per, flops)
    value = st["value"]
    ms_per_step = st["ms_per_step"]
    print(f"[bench] {w.name}: median {ms_per_step:.3f} ms/step (min {st['ms_min']:.3f}, max "
          f"{st['ms_max']:.3f}, bracket mean {bracket_ms / args.steps:.3f}), {value:.1f} TFLOP/s, "
          f"SCLK {clock and clock.get('mhz_median')} MHz (wall {wall:.2f} s for {args.steps} "
          "steps)", file=sys.stderr, flush=True)

    # Per-kernel-class event timing over the same number of steps. While
    # profiling, the library runs the backward on one stream (no overlap of
    # the weight gradients), so each launch group is timed alone. A padding
    # mask's allowed pairs are handed over for the attention classes' FLOPs.
    pairs = (d.seq * int(sum(int(v) for v in vl))) if d.mask == "padding" else 0
    _check("tp_layer_profile", B.tp_layer_profile(sh.handle, 1, pairs))
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    breakdown = {}
    for k in B.KCLASSES:
        rc, n, kms, kfl, kby = B.tp_layer_profile_read(sh.handle, k)
        _check("tp_layer_profile_read", rc)
        if n:
            breakdown[k] = {"launches_per_step": n / args.steps, "ms_per_step": kms / args.steps,
                            "gflop_per_step": kfl / args.steps / 1e9,
                            "gbyte_per_step": kby / args.steps / 1e9}
    B.tp_layer_profile(sh.handle, 0)
    dom = max(breakdown, key=lambda k: breakdown[k]["ms_per_step"])
    bd = breakdown[dom]
    if bd["gflop_per_step"] > 0:
        peak, unit = PEAK[d.dtype]
        achieved = bd["gflop_per_step"] / bd["ms_per_step"]  # GFLOP/ms = TFLOP/s
        roof = {"kernel": dom, "bound": "mfma" if d.dtype == "bf16" else "alu",
                "achieved": achieved, "peak": peak, "unit": unit, "frac": achieved / peak,
                "traffic": stored_traffic(dom, w.name),
                "algorithmic_bytes_per_launch": bd["gbyte_per_step"] * 1e9 / bd["launches_per_step"],
                "algorithmic_flop_per_launch": bd["gflop_per_step"] * 1e9 / bd["launches_per_step"]}
    else:
        achieved = bd["gbyte_per_step"] / bd["ms_per_step"] * 1e3  # GB/s
        roof = {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                "traffic": stored_traffic(dom, w.name),
                "algorithmic_bytes_per_launch": bd["gbyte_per_step"] * 1e9 / bd["launches_per_step"]}
    roof["launches_per_step"] = bd["launches_per_step"]
    roof["avg_launch_ms"] = bd["ms_per_step"] / bd["launches_per_step"]
    roof["timing"] = "HIP events on the launch stream, profiled pass with a serial backward"
    ws_bytes = sh.ws_bytes
    cleanup()
    del step, sh
    torch.cuda.empty_cache()

    others = {}
    if not args.no_other_workloads and args.workload == DEFAULT_WORKLOAD and not sp:
        for name in OTHER_WORKLOADS:
            ow = WORKLOADS[name]
            ostep, osh, ovl, oclean = make_train_step(ow, False, args.recompute,
                                                      overlap=overlap)
            oper, _, _, _ = timed_steps(ostep, max(args.steps, 50), args.warmup)
            ost = step_stats(oper, algorithmic_flops(ow.dims, ovl))
            others[name] = {k: ost[k] for k in ("value", "pct_of_peak", "ms_per_step", "ms_min",
                                                 "ms_max")}
            others[name]["gflop_per_step"] = algorithmic_flops(ow.dims, ovl) / 1e9
            print(f"[bench] {name}: median {ost['ms_per_step']:.3f} ms/step, "
                  f"{ost['value']:.1f} TFLOP/s", file=sys.stderr, flush=True)
            oclean()
            del ostep, osh
            torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_tokens, args.cpu_min_seconds, params)
        print(f"[bench] cpu oracle: {cpu['value'] * 1e3:.1f} GFLOP/s on {cpu['cores']} threads "
              f"({cpu['seconds']:.1f} s; {cpu['sample']})", file=sys.stderr, flush=True)
    del params

    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": d.dtype, "data": "synthetic (seeded N(0,1) inputs, N(0,0.02) weights)",
        "pct_of_peak": st["pct_of_peak"],
        "timing": {"statistic": "median of per-step HIP event pairs", "ms_min": st["ms_min"],
                   "ms_max": st["ms_max"], "ms_mean": st["ms_mean"],
                   "ms_bracket_mean": bracket_ms / args.steps, "wall_s": wall,
                   "sclk": clock},
        "mfma_operands": "fp16" if d.dtype == "bf16" else None,
        "accumulate": "fp32",
        "config": {"workload": w.name, "micro_batch": d.batch, "seq_len": d.seq,
                   "hidden": d.hidden, "heads": d.heads, "ffn": d.ffn, "t": d.t,
                   "rank": w.rank, "mask": d.mask, "gflop_per_step": flops / 1e9,
                   "recompute": "fc1" if args.recompute else "none", "layout": args.layout,
                   "overlap": args.overlap,
                   "workspace_bytes": ws_bytes},
        "roofline": roof, "cpu_baseline": cpu, "breakdown": breakdown,
        "other_workloads": others or None,
    }
    print(json.dumps(line))


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 50; 1000 for --mode decode)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-tokens", type=int, default=512,
                    help="tokens in the oracle's sample (whole sequences, or the first positions "
                         "of a single sequence)")
    ap.add_argument("--cpu-min-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="time only --workload (by default the headline run also times the "
                         "1.2B, 8.3B and BERT 3.9B shards)")
    ap.add_argument("--no-sclk", action="store_true", help="do not sample the GPU clock")
    ap.add_argument("--layout", choices=("tp", "sp"), default="tp",
                    help="tp: TP_ALL forward + backward of one rank; sp: one rank's share of the "
                         "sequence-parallel phases (its kernels only, exchanges excluded)")
    ap.add_argument("--recompute", action="store_true",
                    help="recompute the FC1 pre-activation in backward (TP_RECOMPUTE_FC1)")
    ap.add_argument("--overlap", choices=("auto", "off", "on"), default="auto",
                    help="weight gradients on the handle's second stream (opts.overlap; "
                         "auto: from hidden 8192)")
    ap.add_argument("--mode", choices=("train", "decode"), default="train",
                    help="train: forward + backward (the headline); decode: one decode step")
    ap.add_argument("--cache-len", type=int, default=0,
                    help="decode: KV cache rows per sequence (default: the workload's seq)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain copy of BYTES (counter calibration) and exit")
    args = ap.parse_args()
    if args.steps is None:
        args.steps = 1000 if args.mode == "decode" else 50
    if args.gpus != 1:
        print(f"bench.py: this build runs one GPU only (asked for --gpus {args.gpus}); "
              "multi-GPU tensor parallelism is described in DESIGN.md, not launched.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        copy_probe(args.copy_probe, 10)
        return
    if args.mode == "decode":
        bench_decode(args)
        return
    bench_train(args)


if __name__ == "__main__":
    main()
