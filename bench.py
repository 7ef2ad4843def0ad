#!/usr/bin/env python3
"""Benchmark of the MiniKV-style compressed-KV path on one MI355X.

One step = the whole hot path over one batch of synthetic input, layer by
layer as a model runs it:
  prefill: for every layer, minikv_prefill_select (pass 1: attention output
           + LSE; pass 2: per-key cumulative scores; top-k + recent window)
           and minikv_pack (INT2 keys/values, fp16 residual tail);
  decode:  for every decode step and every layer, minikv_append_decode
           (append the new token -- flushing the residual every 128 tokens --
           and attend over the packed cache plus the residual).
Inputs (prompt Q/K/V of every layer and the decode-step q/k/v, all
distinct, drawn on the device) are resident in HBM before the timed region.

The default workload is the largest single-GPU one: the Llama-3-8B-shaped
131072-token GQA stack (32 layers, 32 query / 8 kv heads, D 128, 64 decode
steps).  The same run adds sub-records for the Llama2-13B-shaped batched
stack (batch 16, 40 heads, 8192 tokens, 256 decode steps) and the
Mistral-7B-shaped GQA stack (batch 4, 32768 tokens, 128 decode steps).

Printed: one JSON line.  `value` is the decode phase's algorithmic bytes
(packed codes + fp16 scale/zero + fp16 residual + q/o, counted as the method
must move them) divided by the decode phase's wall time; the prefill phase's
algorithmic TFLOP/s (3 D n (n+1) per query head and layer: QK^T and PV of
pass 1, QK^T again in pass 2) is reported next to it.  `roofline` is for the
decode-attention call and `roofline_prefill` for the prefill+select call,
each timed with HIP events on the stream it runs on.  `cpu_baseline` times
the CPU oracle on a bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
MFMA_FP16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 MFMA, published
HEADLINE_CONFIG = 5


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=3)
    p.add_argument("--warmup", type=int, default=1)
    p.add_argument("--config", type=int, default=HEADLINE_CONFIG,
                   help="workload id (configs.py); default: the 131072-token "
                        "Llama-3-8B-shaped GQA stack, the largest that fits "
                        "one GPU")
    p.add_argument("--sub-configs", default="3,4,2",
                   help="comma-separated workloads measured after the "
                        "headline one, one sub-record each ('' for none)")
    p.add_argument("--sub-steps", type=int, default=1)
    p.add_argument("--distinct-layers", type=int, default=0,
                   help="generate this many distinct layer inputs and cycle "
                        "them (0 = all layers distinct)")
    p.add_argument("--distinct-steps", type=int, default=0,
                   help="distinct decode-step inputs to generate and cycle "
                        "(0 = all)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--eager", action="store_true",
                   help="launch every call from Python instead of replaying "
                        "the captured HIP graphs of a step")
    p.add_argument("--decode-probe", type=int, default=0, metavar="N",
                   help="run only the decode-call timing at layer 0 of "
                        "workload N (two alternating caches) and print it")
    p.add_argument("--prefill-probe", type=int, default=0, metavar="N",
                   help="run only layer 0's prefill+select call of workload "
                        "N, twice (the workload of the MFMA counters)")
    p.add_argument("--traffic-probe", type=int, default=0, metavar="N",
                   help="run only the short workload whose HBM counters "
                        "(rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE) give the "
                        "decode roofline's traffic at workload N: a 256 MiB "
                        "device copy for calibration, then one decode call "
                        "per layer at the end-of-step cache state")
    p.add_argument("--no-persistence", action="store_true",
                   help="skip the persistence audit (re-selection every 32 "
                        "decode steps, overlap with the prefill heavy "
                        "hitters)")
    p.add_argument("--no-mixed", action="store_true",
                   help="skip the MiKV / DiffKV mixed-precision records")
    p.add_argument("--no-fused-tail", action="store_true",
                   help="skip the fused prefill tail record")
    p.add_argument("--mixed-configs", default="5,3",
                   help="workloads of the mixed-precision records (layer 0)")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="rough CPU budget of the oracle baseline")
    return p.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# ------------------------------------------------------------ accounting --

def decode_bytes(c, n_packed, n_res):
    """Algorithmic bytes of one decode-attention call (all units)."""
    D, Gk, Gv = c["D"], c["Gk"], c["Gv"]
    units = c["B"] * c["Hkv"]
    per_unit = (n_packed * D // 4 * 2                      # K and V codes
                + (n_packed // Gk) * D * 4                  # K scale+zero
                + n_packed * (D // Gv) * 4                  # V scale+zero
                + n_res * D * 4)                            # fp16 residual
    return units * per_unit + c["B"] * c["Hq"] * D * 4      # + q and o


def prefill_flops(c):
    n, D = c["n"], c["D"]
    return 3.0 * D * n * (n + 1) * c["B"] * c["Hq"]


def budgets(mk, c):
    return mk.pyramid_budgets(c["n"], c["L"], c["hh"], c["rw"], c["depth"],
                              c["pyramid"])


def layer_capacity(c, m):
    Gk, nr, S = c["Gk"], c["residual_cap"], c["decode_steps"]
    return ((m // Gk) * Gk + S + nr + Gk - 1) // Gk * Gk


# ------------------------------------------------------- traffic summary --

def traffic_file(config_id):
    from bit_quantized_attention_two_amd import configs
    return os.path.join(ROOT, "profiles", "decode_%s_traffic.md" %
                        configs.get(config_id)["name"].replace("-", "_"))


DECODE_SRC = os.path.join(ROOT, "bit_quantized_attention_two_amd", "csrc",
                          "decode.hip")


def measured_traffic(config_id):
    """HBM bytes per decode call from the committed counter summary, or None
    when there is none for this workload or the decode source has changed
    since the counters were taken."""
    import hashlib
    path = traffic_file(config_id)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("|", "#", " ")):
            k, _, v = line.partition(":")
            fields[k.strip()] = v.strip()
    h = hashlib.sha256(open(DECODE_SRC, "rb").read()).hexdigest()
    if fields.get("decode_source_sha256") != h:
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ------------------------------------------------------------------ probes --

def traffic_probe(config_id):
    """Workload of the traffic counters (see --traffic-probe)."""
    import torch
    from bit_quantized_attention_two_amd import configs, minikv
    c = configs.get(config_id)
    B, Hq, Hkv, D, n, L = c["B"], c["Hq"], c["Hkv"], c["D"], c["n"], c["L"]
    ks, r = budgets(minikv, c)
    dims = minikv.make_dims(B, Hq, Hkv, D, c["Gk"], c["Gv"], c["residual_cap"])
    g = torch.Generator(device="cuda").manual_seed(11)
    src = torch.randn(64 * 1024 * 1024, device="cuda", generator=g)  # 256 MiB
    dst = torch.empty_like(src)
    k = torch.randn(B, Hkv, n, D, device="cuda", generator=g).half()
    v = torch.randn(B, Hkv, n, D, device="cuda", generator=g).half()
    kn = torch.randn(B, Hkv, D, device="cuda", generator=g).half()
    nr, Gk = c["residual_cap"], c["Gk"]
    caches = []
    for l in range(L):
        # the end-of-step state: the selection plus the decode steps'
        # tokens, flushed every nr, packed directly (appends under the
        # counters would each be a profiled dispatch); the residual's count
        # is set on the host (its contents do not change the traffic)
        m = ks[l] + r
        n_res = m % Gk
        n_packed = m - n_res
        for _ in range(c["decode_steps"]):
            n_res += 1
            if n_res == nr:
                n_packed, n_res = n_packed + nr, 0
        sel = (torch.arange(n_packed, device="cuda", dtype=torch.int64) * n //
               n_packed).int().repeat(B, Hkv, 1).contiguous()
        cache = minikv.LayerCache(dims, layer_capacity(c, m))
        minikv.pack(dims, k, v, sel, cache)
        cache.c.n_res = n_res
        caches.append(cache)
    del k, v
    q = torch.randn(B, Hq, D, device="cuda", generator=g).half()
    o = torch.empty_like(q)
    ws = torch.zeros(minikv.decode_ws_bytes(dims, max(x.capacity for x in caches)),
                     dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    alg = 0
    for cache in caches:
        minikv.decode_attn(dims, cache, q, o, ws)
        alg += decode_bytes(c, cache.n_packed, cache.n_res)
    torch.cuda.synchronize()
    print(json.dumps({"workload": c["name"], "copy_bytes": src.numel() * 4,
                      "decode_calls": L,
                      "algorithmic_bytes_per_call": alg / L}), flush=True)


def prefill_probe(config_id):
    """Layer 0's prefill+select call of a workload, twice, for counters."""
    import torch
    from bit_quantized_attention_two_amd import configs, minikv, synth
    c = configs.get(config_id)
    ks, r = budgets(minikv, c)
    dims = minikv.make_dims(c["B"], c["Hq"], c["Hkv"], c["D"], c["Gk"],
                            c["Gv"], c["residual_cap"])
    q, k, v = synth.gen_prefill_device(config_id, 0, "cuda", c)
    for _ in range(2):
        minikv.prefill_select(dims, q, k, v, ks[0], r)
    torch.cuda.synchronize()
    print(json.dumps({"workload": c["name"], "calls": 2,
                      "algorithmic_flops_per_call": prefill_flops(c)}),
          flush=True)


def layer_decode_roofline(stream, config_id):
    """Decode-attention call at layer 0 of a workload: its heavy-hitter
    budget plus the recent window packed, then 64 tokens in the fp16
    residual.  Two such caches alternate (no call finds the previous call's
    data in the last-level cache at the large workloads), timed as a graph of
    back-to-back calls between HIP events on `stream`: 10 replays to warm up
    (the clock ramps up under sustained load), then the median of 10."""
    import torch
    from bit_quantized_attention_two_amd import configs, minikv
    c = configs.get(config_id)
    B, Hq, Hkv, D, n = c["B"], c["Hq"], c["Hkv"], c["D"], c["n"]
    dims = minikv.make_dims(B, Hq, Hkv, D, c["Gk"], c["Gv"], c["residual_cap"])
    ks, r = budgets(minikv, c)
    m, res = ks[0] + r, 64
    g = torch.Generator(device="cuda").manual_seed(3)
    k = torch.randn(B, Hkv, n, D, device="cuda", generator=g).half()
    v = torch.randn(B, Hkv, n, D, device="cuda", generator=g).half()
    sel = (torch.arange(m, device="cuda", dtype=torch.int64) * n // m
           ).int().repeat(B, Hkv, 1).contiguous()
    caches = []
    for i in range(2):
        cache = minikv.LayerCache(dims, (m // c["Gk"]) * c["Gk"] + 256)
        minikv.pack(dims, k, v, (sel + i) % n, cache)
        for t in range(res - cache.n_res):       # decode-step tokens
            minikv.append(dims, cache, k[:, :, t].contiguous(),
                          v[:, :, t].contiguous())
        caches.append(cache)
    del k, v
    n_packed = caches[0].n_packed
    q = torch.randn(B, Hq, D, device="cuda", generator=g).half()
    o = torch.empty_like(q)
    ws = torch.zeros(minikv.decode_ws_bytes(dims, caches[0].capacity),
                     dtype=torch.uint8, device="cuda")
    R = 20
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        minikv.decode_attn(dims, caches[0], q, o=o, ws=ws)
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=side):
            for i in range(R):
                minikv.decode_attn(dims, caches[i % 2], q, o=o, ws=ws)
    stream.wait_stream(side)
    for _ in range(10):
        gr.replay()
    ev = [(torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(10)]
    for a, b in ev:
        a.record(stream)
        gr.replay()
        b.record(stream)
    torch.cuda.synchronize()
    us = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3 / R
    alg = decode_bytes(c, n_packed, res)
    achieved = alg / (us * 1e-6) / 1e9
    return {"kernel": "minikv_decode_attn (split-KV decode + combine "
                      "kernels)",
            "workload": "%s layer 0: batch %d, %d kv heads, g %d, D %d, %d "
                        "packed + %d residual tokens per kv head" % (
                            c["name"], B, Hkv, Hq // Hkv, D, n_packed, res),
            "bound": "hbm", "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "avg_launch_us": round(us, 3),
            "algorithmic_bytes_per_launch": int(alg), "launches": R}


# --------------------------------------------------------------- workload --

def run_workload(cfg_id, steps, warmup, args, stream, headline):
    """Generate a workload's inputs on the device, time `steps` whole steps
    (two HIP graphs each: prefill part, decode part) and the per-call
    rooflines.  Returns (record, state) where state keeps what the
    persistence audit and the CPU baseline reuse."""
    import torch
    from bit_quantized_attention_two_amd import configs, minikv, synth
    c = configs.get(cfg_id)
    dev = torch.device("cuda:0")
    B, Hq, Hkv, D, n, L = c["B"], c["Hq"], c["Hkv"], c["D"], c["n"], c["L"]
    Gk, Gv, nr, S = c["Gk"], c["Gv"], c["residual_cap"], c["decode_steps"]
    ks, r = budgets(minikv, c)
    dims = minikv.make_dims(B, Hq, Hkv, D, Gk, Gv, nr)
    nl = args.distinct_layers or L
    ns = args.distinct_steps or S

    t0 = time.time()
    qkv = [synth.gen_prefill_device(cfg_id, l, dev, c) for l in range(nl)]
    dq, dk, dv = synth.gen_decode_device(cfg_id, ns, nl, dev, c)
    torch.cuda.synchronize()
    gen_s = time.time() - t0
    log("%s: inputs generated in %.1f s" % (c["name"], gen_s))

    caches, sels, cols = [], [], []
    out = torch.empty((B, Hq, n, D), dtype=torch.float16, device=dev)
    ws_pref = torch.empty(minikv.prefill_ws_bytes(dims, n), dtype=torch.uint8,
                          device=dev)
    for l in range(L):
        m = ks[l] + r
        caches.append(minikv.LayerCache(dims, layer_capacity(c, m), dev))
        cols.append(torch.empty((B, Hkv, n), dtype=torch.float32, device=dev))
        sels.append(torch.empty((B, Hkv, m), dtype=torch.int32, device=dev))
    max_cap = max(x.capacity for x in caches)
    ws_dec = torch.zeros(minikv.decode_ws_bytes(dims, max_cap),
                         dtype=torch.uint8, device=dev)
    od = torch.empty((B, Hq, D), dtype=torch.float16, device=dev)
    dec_bytes_per_call = []

    def prefill_part():
        for l in range(L):
            q, k, v = qkv[l % nl]
            minikv.prefill_select(dims, q, k, v, ks[l], r, o=out,
                                  col=cols[l], sel=sels[l], ws=ws_pref)
            minikv.pack(dims, k, v, sels[l], caches[l])

    def decode_part():
        dec_bytes_per_call.clear()
        for s in range(S):
            for l in range(L):
                cache = caches[l]
                minikv.append_decode(dims, cache, dk[s % ns, l % nl],
                                     dv[s % ns, l % nl], dq[s % ns, l % nl],
                                     o=od, ws=ws_dec)
                dec_bytes_per_call.append(decode_bytes(c, cache.n_packed,
                                                       cache.n_res))

    def capture(fn, side):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            fn()
        return g

    for _ in range(max(1, warmup)):
        prefill_part()
        decode_part()
    torch.cuda.synchronize()
    log("%s: eager warm-up done" % c["name"])
    side = torch.cuda.Stream()
    graphs = None
    if not args.eager:
        side.wait_stream(stream)
        graphs = (capture(prefill_part, side), capture(decode_part, side))
        stream.wait_stream(side)
        for _ in range(warmup):
            graphs[0].replay()
            graphs[1].replay()
        torch.cuda.synchronize()
        log("%s: graphs captured" % c["name"])

    phase = []
    t_start = time.perf_counter()
    for _ in range(steps):
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        e0.record(stream)
        graphs[0].replay() if graphs else prefill_part()
        e1.record(stream)
        graphs[1].replay() if graphs else decode_part()
        e2.record(stream)
        phase.append((e0, e1, e2, sum(dec_bytes_per_call)))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    log("%s: %d timed steps in %.1f s" % (c["name"], steps, wall))

    # Per-call durations of the two dominant calls, right after the timed
    # steps, on the same stream, with HIP events: every layer's decode call
    # in its end-of-step cache state, replayed back-to-back from a graph (R
    # rounds of all layers); each layer's decode call on its own; each
    # layer's prefill+select call between its own events.
    R = 8
    ka, kb = (torch.cuda.Event(enable_timing=True) for _ in range(2))

    def timed_graph(fn):
        side.wait_stream(stream)
        g_ = capture(fn, side)
        stream.wait_stream(side)
        g_.replay()
        ka.record(stream)
        g_.replay()
        kb.record(stream)
        torch.cuda.synchronize()
        return ka.elapsed_time(kb)

    dec_call_ms = timed_graph(lambda: [
        minikv.decode_attn(dims, caches[l], dq[0, l % nl], o=od, ws=ws_dec)
        for _ in range(R) for l in range(L)]) / (R * L)
    layer_us = [timed_graph(lambda: [
        minikv.decode_attn(dims, caches[l], dq[0, l % nl], o=od, ws=ws_dec)
        for _ in range(R)]) * 1e3 / R for l in range(L)]
    mass_rec = None
    if headline:
        mass = torch.zeros((B, Hkv, max_cap + nr), dtype=torch.float32,
                           device=dev)
        ws_mass = torch.empty(minikv.decode_mass_ws_bytes(dims, max_cap),
                              dtype=torch.uint8, device=dev)
        mass_ms = timed_graph(lambda: [
            minikv.decode_attn_mass(dims, caches[l], dq[0, l % nl], mass,
                                    o=od, ws=ws_mass)
            for _ in range(R) for l in range(L)]) / (R * L)
        mass_rec = {"kernel": "minikv_decode_attn_mass (decode + per-token "
                              "attention mass, accumulated)",
                    "avg_launch_us": round(mass_ms * 1e3, 3),
                    "vs_decode_call": round(mass_ms / dec_call_ms, 3)}
        del mass, ws_mass
    dec_call_bytes = np.array([decode_bytes(c, x.n_packed, x.n_res)
                               for x in caches], np.float64)
    pre_ev = []
    for l in range(L):
        q, k, v = qkv[l % nl]
        a, b = (torch.cuda.Event(enable_timing=True) for _ in range(2))
        a.record(stream)
        minikv.prefill_select(dims, q, k, v, ks[l], r, o=out, col=cols[l],
                              sel=sels[l], ws=ws_pref)
        b.record(stream)
        pre_ev.append((a, b))
    torch.cuda.synchronize()
    pre_call_ms = np.array([a.elapsed_time(b) for a, b in pre_ev])

    pre_ms = sum(e0.elapsed_time(e1) for e0, e1, _, _ in phase)
    dec_ms = sum(e1.elapsed_time(e2) for _, e1, e2, _ in phase)
    dec_bytes = sum(x[3] for x in phase)
    value = dec_bytes / (dec_ms * 1e-3) / 1e9
    pre_tflops = prefill_flops(c) * L * steps / (pre_ms * 1e-3) / 1e12
    avg_dec_bytes = float(dec_call_bytes.mean())
    achieved = avg_dec_bytes / (dec_call_ms * 1e-3) / 1e9
    pre_achieved = prefill_flops(c) / (pre_call_ms.mean() * 1e-3) / 1e12
    traffic = measured_traffic(cfg_id)

    rec = {
        "workload": c["name"],
        "decode_gbs": round(value, 2),
        "decode_pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "prefill_tflops": round(pre_tflops, 2),
        "prefill_pct_mfma_fp16_peak": round(100 * pre_tflops /
                                            MFMA_FP16_PEAK_TFLOPS, 2),
        "ms_per_step": round(wall * 1e3 / steps, 3),
        "steps": steps,
        "phase_ms_per_step": {"prefill": round(pre_ms / steps, 3),
                              "decode": round(dec_ms / steps, 3)},
        "config": {
            "workload": c["name"], "config_id": cfg_id, "batch": B,
            "n_q_heads": Hq, "n_kv_heads": Hkv, "head_dim": D,
            "prompt_len": n, "layers": L, "decode_steps": S,
            "budget": "pyramid d=%d" % c["depth"] if c["pyramid"] else
                      "uniform", "hh_frac": "1/4", "recent_frac": "1/4",
            "group_k": Gk, "group_v": Gv, "residual_cap": nr,
            "distinct_layer_inputs": nl, "distinct_decode_inputs": ns,
            "parallelism": "single GPU",
            "launch": "eager" if args.eager else
                      "HIP graphs (one step captured, replayed per step)",
        },
        "roofline": {
            "kernel": "minikv_decode_attn (split-KV decode + combine "
                      "kernels), all layers, end-of-step cache state",
            "bound": "hbm", "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "traffic_ratio": round(traffic / avg_dec_bytes, 4)
            if traffic else None,
            "avg_launch_us": round(dec_call_ms * 1e3, 3),
            "algorithmic_bytes_per_launch": int(avg_dec_bytes),
            "launches": R * L,
            "per_layer_call_us": {
                "median": round(float(np.median(layer_us)), 3),
                "p90": round(float(np.percentile(layer_us, 90)), 3),
                "min": round(min(layer_us), 3),
                "max": round(max(layer_us), 3)},
        },
        "roofline_prefill": {
            "kernel": "minikv_prefill_select (pass 1 + pass 2 + select), "
                      "every layer",
            "bound": "mfma", "achieved": round(pre_achieved, 2),
            "peak": MFMA_FP16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(pre_achieved / MFMA_FP16_PEAK_TFLOPS, 4),
            "avg_launch_us": round(float(pre_call_ms.mean()) * 1e3, 3),
            "algorithmic_flops_per_launch": prefill_flops(c),
            # context only: the FlashAttention convention counts pass 1's
            # 2 D n (n+1) per query head and not the score pass
            "achieved_pass1_convention": round(pre_achieved * 2 / 3, 2),
        },
        "input_generation_s": round(gen_s, 1),
    }
    if mass_rec:
        rec["decode_mass_audit"] = mass_rec
    if avg_dec_bytes < 64e6 and dec_call_ms * 1e3 < 20:
        rec["roofline"]["regime"] = ("launch-bound: about %.0f MB per call, "
                                     "timed as a graph of every layer's call"
                                     % (avg_dec_bytes / 1e6))
    state = dict(c=c, ks=ks, r=r, dims=dims, qkv=qkv, dq=dq, dk=dk, dv=dv)
    del graphs, caches, cols, sels, out, ws_pref, ws_dec
    return rec, state


def mixed_decode_bytes(c, segs, n_res):
    """Algorithmic bytes of one mixed-precision decode call: per unit and
    segment, (key_bits + value_bits) D / 8 code bytes per packed token plus
    fp16 scale and zero (per key group and channel, per token and value
    group), the fp16 residual, and q and o.  segs: (key_bits, value_bits,
    total packed tokens over all units)."""
    D, Gk, Gv = c["D"], c["Gk"], c["Gv"]
    total = 0
    for kb, vb, tokens in segs:
        total += tokens * (kb + vb) * D // 8 + (tokens // Gk) * D * 4 + \
            tokens * (D // Gv) * 4
    units = c["B"] * c["Hkv"]
    return total + units * n_res * D * 4 + c["B"] * c["Hq"] * D * 4


def mixed_records(stream, config_id, alphas=(1.0, 0.04)):
    """MiKV and DiffKV at layer 0 of a workload, on its device-drawn inputs:
      MiKV: the library's heavy-hitter + recent-window selection marks the
        important tokens; minikv_pack_mikv keeps them at INT4 and every
        other prompt token at INT2 (average 3 bits at a half/half split);
      DiffKV: minikv_prefill_diffkv (pass 1 + the per-head significance
        pass), minikv_tier_diffkv (alpha_hi, alpha_lo), minikv_pack_diffkv
        (K8V4 / K4V2, per kv head).
    Each then gets 64 decode-step tokens in the fp16 residual, and its
    decode call is timed like the layer call of layer_decode_roofline: two
    caches with the same contents alternate in a graph of 20 calls (more
    than the last-level cache at these sizes), 10 warm-up replays, median
    of 10.  Pack, prefill and tier calls are timed between HIP events."""
    import torch
    from bit_quantized_attention_two_amd import configs, minikv, synth
    c = configs.get(config_id)
    B, Hq, Hkv, D, n = c["B"], c["Hq"], c["Hkv"], c["D"], c["n"]
    Gk = c["Gk"]
    dims = minikv.make_dims(B, Hq, Hkv, D, Gk, 16, c["residual_cap"])
    ks, r = budgets(minikv, c)
    m = int(ks[0]) + r
    q, k, v = synth.gen_prefill_device(config_id, 0, "cuda", c)
    dq, dk, dv = synth.gen_decode_device(config_id, 64, 1, "cuda", c)
    ev = lambda: (torch.cuda.Event(enable_timing=True),
                  torch.cuda.Event(enable_timing=True))

    def timed(fn):
        a, b = ev()
        a.record(stream)
        out = fn()
        b.record(stream)
        torch.cuda.synchronize()
        return out, a.elapsed_time(b)

    def decode_time(caches):
        o = torch.empty((B, Hq, D), dtype=torch.float16, device="cuda")
        ws = torch.zeros(minikv.decode_mixed_ws_bytes(dims, caches[0]),
                         dtype=torch.uint8, device="cuda")
        R = 20
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            minikv.decode_mixed(dims, caches[0], dq[0, 0], o=o, ws=ws)
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=side):
                for i in range(R):
                    minikv.decode_mixed(dims, caches[i % 2], dq[0, 0], o=o, ws=ws)
        stream.wait_stream(side)
        for _ in range(10):
            gr.replay()
        ts = []
        for _ in range(10):
            a, b = ev()
            a.record(stream)
            gr.replay()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts)) * 1e3 / R

    def fill_residual(cache):
        for t in range(64 - cache.n_res):
            minikv.append_mixed(dims, cache, dk[t, 0], dv[t, 0])

    recs = {}
    # ---- MiKV
    _, _, sel = minikv.prefill_select(dims, q, k, v, int(ks[0]), r)
    segs = [(4, 4, (m // Gk) * Gk + 256), (2, 2, ((n - m) // Gk) * Gk + Gk)]
    caches, pack_ms = [], []
    for _ in range(2):
        mc = minikv.MixedCache(dims, segs, flush_seg=0)
        _, ms = timed(lambda: minikv.pack_mikv(dims, k, v, sel, mc))
        pack_ms.append(ms)
        fill_residual(mc)
        caches.append(mc)
    units = B * Hkv
    seg_tok = [(4, 4, caches[0].n_packed(0) * units), (2, 2, caches[0].n_packed(1) * units)]
    alg = mixed_decode_bytes(c, seg_tok, caches[0].n_res)
    us = decode_time(caches)
    recs["mikv"] = {
        "workload": "%s layer 0: %d kv heads x (%d INT4 + %d INT2 packed + %d fp16 "
                    "residual tokens)" % (c["name"], units, caches[0].n_packed(0),
                                          caches[0].n_packed(1), caches[0].n_res),
        "decode": {"bound": "hbm", "achieved": round(alg / (us * 1e-6) / 1e9, 2),
                   "peak": HBM_PEAK_GBS, "unit": "GB/s",
                   "frac": round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                   "avg_launch_us": round(us, 3), "algorithmic_bytes_per_launch": alg},
        "pack_mikv_ms": round(min(pack_ms), 3),
        "average_code_bits": round(sum(kb * t for kb, _, t in seg_tok) /
                                   max(1, sum(t for _, _, t in seg_tok)), 3),
    }
    del caches, sel
    torch.cuda.empty_cache()
    # ---- DiffKV
    score = torch.empty((B, Hkv, n), dtype=torch.float32, device="cuda")
    o_pre = torch.empty_like(q)
    ws_pre = torch.empty(minikv.prefill_ws_bytes(dims, n), dtype=torch.uint8,
                         device="cuda")
    minikv.prefill_diffkv(dims, q, k, v, o=o_pre, score=score, ws=ws_pre)
    _, pre_ms = timed(lambda: minikv.prefill_diffkv(dims, q, k, v, o=o_pre, score=score,
                                                    ws=ws_pre))
    tiers, tier_ms = timed(lambda: minikv.tier_diffkv(dims, score, *alphas))
    idx_hi, idx_lo, n_hi, n_lo = tiers
    bound = n // Gk * Gk
    nh, nl = n_hi.cpu().numpy(), n_lo.cpu().numpy()
    dsegs = [(8, 4, bound), (4, 2, bound), (8, 4, 256)]
    caches, pack_ms = [], []
    for _ in range(2):
        mc = minikv.MixedCache(dims, dsegs, flush_seg=2)
        _, ms = timed(lambda: minikv.pack_diffkv(dims, k, v, idx_hi, idx_lo, n_hi, n_lo, mc))
        pack_ms.append(ms)
        # the host reads the per-head counts back once and narrows the grid
        mc.set_bound(0, int(nh.max()))
        mc.set_bound(1, int(nl.max()))
        fill_residual(mc)
        caches.append(mc)
    seg_tok = [(8, 4, int(nh.sum())), (4, 2, int(nl.sum()))]
    alg = mixed_decode_bytes(c, seg_tok, caches[0].n_res)
    us = decode_time(caches)
    pre_fl = prefill_flops(c)
    recs["diffkv"] = {
        "workload": "%s layer 0: %d kv heads, alpha_hi %g, alpha_lo %g" % (
            c["name"], units, alphas[0], alphas[1]),
        "tier_tokens_per_kv_head": {"k8v4": nh.tolist(), "k4v2": nl.tolist(),
                                    "pruned": (n - nh - nl).tolist()},
        "prefill": {"bound": "mfma", "achieved": round(pre_fl / (pre_ms * 1e-3) / 1e12, 2),
                    "peak": MFMA_FP16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(pre_fl / (pre_ms * 1e-3) / 1e12 / MFMA_FP16_PEAK_TFLOPS, 4),
                    "call_ms": round(pre_ms, 3), "algorithmic_flops_per_launch": pre_fl},
        "tier_ms": round(tier_ms, 3),
        "pack_diffkv_ms": round(min(pack_ms), 3),
        "decode": {"bound": "hbm", "achieved": round(alg / (us * 1e-6) / 1e9, 2),
                   "peak": HBM_PEAK_GBS, "unit": "GB/s",
                   "frac": round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                   "avg_launch_us": round(us, 3), "algorithmic_bytes_per_launch": alg},
    }
    return recs


def fused_tail_record(stream, config_id, reps=5):
    """Layer 0 of a workload: minikv_prefill_select followed by minikv_pack,
    against minikv_prefill_select_pack with the selection inside the second
    prefill pass (fused) and after it; each a graph of one layer's calls
    timed between HIP events, alternated `reps` times; medians."""
    import torch
    from bit_quantized_attention_two_amd import configs, minikv, synth
    c = configs.get(config_id)
    B, Hq, Hkv, D, n = c["B"], c["Hq"], c["Hkv"], c["D"], c["n"]
    ks, r = budgets(minikv, c)
    n_hh, m = int(ks[0]), int(ks[0]) + r
    dims = minikv.make_dims(B, Hq, Hkv, D, c["Gk"], c["Gv"], c["residual_cap"])
    q, k, v = synth.gen_prefill_device(config_id, 0, "cuda", c)
    o = torch.empty_like(q)
    col = torch.empty((B, Hkv, n), dtype=torch.float32, device="cuda")
    sel = torch.empty((B, Hkv, m), dtype=torch.int32, device="cuda")
    cache = minikv.LayerCache(dims, (m // c["Gk"]) * c["Gk"] + c["Gk"])
    ws1 = torch.empty(minikv.prefill_ws_bytes(dims, n), dtype=torch.uint8, device="cuda")
    ws2 = torch.empty(minikv.prefill_tail_ws_bytes(dims, n), dtype=torch.uint8,
                      device="cuda")

    def separate():
        minikv.prefill_select(dims, q, k, v, n_hh, r, o=o, col=col, sel=sel, ws=ws1)
        minikv.pack(dims, k, v, sel, cache)

    def fused():
        minikv.prefill_select_pack(dims, q, k, v, n_hh, r, cache, fuse_select=True, o=o,
                                   col=col, sel=sel, ws=ws2)

    def one_call():
        minikv.prefill_select_pack(dims, q, k, v, n_hh, r, cache, fuse_select=False, o=o,
                                   col=col, sel=sel, ws=ws2)

    graphs = []
    side = torch.cuda.Stream()
    for fn in (separate, fused, one_call):
        fn()
        side.wait_stream(stream)
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=side):
            fn()
        stream.wait_stream(side)
        graphs.append(gr)
    ts = [[], [], []]
    for _ in range(reps):
        for i, gr in enumerate(graphs):
            a, b = (torch.cuda.Event(enable_timing=True) for _ in range(2))
            a.record(stream)
            gr.replay()
            b.record(stream)
            torch.cuda.synchronize()
            ts[i].append(a.elapsed_time(b) * 1e3)
    sep, fus, one = (float(np.median(t)) for t in ts)
    return {"workload": "%s layer 0 (%d units, %d selected of %d)" % (
                c["name"], B * Hkv, m, n),
            "separate_calls_us": round(sep, 2),
            "one_call_selection_kernel_us": round(one, 2),
            "one_call_fused_selection_us": round(fus, 2),
            "fused_saved_pct": round(100 * (sep - fus) / sep, 2)}


def persistence_audit(st, layer=0, every=32):
    """The persistence test the MiniKV verdict record's falsifier asks for,
    on this workload's synthetic inputs: would the heavy hitters chosen at
    the end of prefill still be chosen later in decoding?  H2O's cumulative
    score at decode step s is the column sum of causal attention over the
    prompt plus the first s generated tokens (their q, k, v are the decode
    steps' inputs), so the selection that step s would make is the library's
    own prefill+select over that extended sequence, with the candidates kept
    to the prompt's [0, n - r) (recent window r + s).  Reported: the mean
    and minimum over kv heads of |HH_s ∩ HH_0| / k every `every` steps, and
    the time of one re-selection at the last step."""
    import torch
    from bit_quantized_attention_two_amd import minikv
    c, ks, r, dims = st["c"], st["ks"], st["r"], st["dims"]
    B, Hkv, n, S = c["B"], c["Hkv"], c["n"], c["decode_steps"]
    n_hh = int(ks[layer])
    q, k, v = st["qkv"][layer]
    ns = st["dq"].shape[0]
    steps = [s % ns for s in range(S)]
    ext = [torch.cat([x, y[steps, layer].permute(1, 2, 0, 3)], dim=2)
           for x, y in ((q, st["dq"]), (k, st["dk"]), (v, st["dv"]))]
    points = list(range(0, S + 1, every))
    if points[-1] != S:
        points.append(S)
    hh0, rows, ms = None, [], 0.0
    for t in points:
        sub = [x[:, :, :n + t].contiguous() for x in ext]
        a, b = (torch.cuda.Event(enable_timing=True) for _ in range(2))
        a.record()
        _, _, sel = minikv.prefill_select(dims, *sub, n_hh, r + t)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        hh = sel[..., :n_hh].cpu().numpy().reshape(B * Hkv, n_hh)
        del sub
        if hh0 is None:
            hh0 = hh
        ov = np.array([np.intersect1d(x, y).size for x, y in zip(hh, hh0)]) / n_hh
        rows.append((t, float(ov.mean()), float(ov.min())))
    return {"layer": layer, "heavy_hitters": n_hh, "recent": r,
            "steps": [x[0] for x in rows],
            "overlap_mean": [round(x[1], 4) for x in rows],
            "overlap_min": [round(x[2], 4) for x in rows],
            "reselect_ms_at_last_step": round(ms, 3)}


def cpu_baseline(st, budget_s):
    """The oracle, as it is, on host threads, on a bounded sample of layer
    0 of the workload (batch element 0, the same device-drawn inputs copied
    to the host): prefill rows (a spread of query rows of one kv head's
    group, O, LSE and their column contributions), the oracle's selection
    from those partial scores, pack of every kv head, and decode attention
    of every kv head repeated for about half the budget.  Reported in the
    metric's unit (decode GB/s) with the prefill row rate next to it."""
    import concurrent.futures as cf

    import oracle
    oracle.build(force=False)
    c, ks, r = st["c"], st["ks"], st["r"]
    host_cores = os.cpu_count() or 1
    cores = min(16, host_cores)          # one GPU's share of the host CPUs
    Hq, Hkv, D, n = c["Hq"], c["Hkv"], c["D"], c["n"]
    g = Hq // Hkv
    q, k, v = (x[0:1].cpu().numpy() for x in st["qkv"][0])
    qd = st["dq"][0, 0].cpu().numpy()
    # prefill: `cores` slices of rows spread over [0, n), one per thread
    rows_per = max(1, int(64 * (131072 / n)) // cores + 1)
    rr = np.random.default_rng(5)
    slices = [np.sort(rr.choice(n, min(rows_per, n), replace=False)).astype(np.int32)
              for _ in range(cores)]
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(cores) as ex:
        parts = list(ex.map(lambda rows: oracle.prefill_rows(
            q[0, :g], k[0, 0], v[0, 0], rows), slices))
    t_pref = time.perf_counter() - t0
    row_flops = sum(float(g * D * 3 * (rows + 1).sum()) * 2 for rows in slices)
    col = np.sum([p[2] for p in parts], axis=0)
    sel0 = oracle.select(col, int(ks[0]), r)
    m = sel0.size
    cap = (m // c["Gk"]) * c["Gk"] + 256
    oc = oracle.OracleCache(1, Hkv, D, c["Gk"], c["Gv"], cap, c["residual_cap"])
    t0 = time.perf_counter()
    oc.pack(k, v, np.tile(sel0, (1, Hkv, 1)), workers=cores)
    t_pack = time.perf_counter() - t0
    nbytes_call = decode_bytes(dict(c, B=1), oc.n_packed, oc.n_res)
    units = list(range(Hkv))
    reps = 0
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(cores) as ex:
        while True:
            list(ex.map(lambda h: oc.decode_unit(qd[0, h * g:(h + 1) * g], 0, h),
                        units))
            reps += 1
            if time.perf_counter() - t0 > budget_s / 2 or reps >= 10000:
                break
    t_dec = time.perf_counter() - t0
    return {
        "value": round(nbytes_call * reps / t_dec / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "host_cores": host_cores,
        "kind": "oracle",
        "sample": "%s layer 0, batch element 0: decode attention of all %d "
                  "kv heads (%d packed + %d residual tokens each) repeated %d "
                  "times on %d threads; before it, %d prefill query rows of "
                  "kv head 0's %d query heads, the oracle's selection from "
                  "their scores, and pack of every kv head; fp64 oracle" %
                  (c["name"], Hkv, oc.n_packed, oc.n_res, reps, cores,
                   sum(s.size for s in slices), g),
        "prefill_rows_tflops": round(row_flops / t_pref / 1e12, 6),
        "pack_s_all_kv_heads": round(t_pack, 3),
        "seconds": round(t_dec + t_pref + t_pack, 2),
    }


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU "
              "path (each GPU would run the same kernels on its own share of "
              "kv heads, with no exchange); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from bit_quantized_attention_two_amd import minikv
    minikv.lib()
    assert torch.cuda.is_available(), "needs a GPU"
    torch.cuda.set_device(0)
    if args.traffic_probe:
        traffic_probe(args.traffic_probe)
        return
    if args.prefill_probe:
        prefill_probe(args.prefill_probe)
        return
    if args.decode_probe:
        print(json.dumps(layer_decode_roofline(torch.cuda.current_stream(),
                                               args.decode_probe)), flush=True)
        return
    stream = torch.cuda.current_stream()

    rec, st = run_workload(args.config, args.steps, args.warmup, args, stream,
                           headline=True)
    result = {
        "metric": "packed-KV decode attention GB/s (% HBM peak) + prefill "
                  "selective-attn TFLOP/s",
        "value": rec["decode_gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 in, fp32 accumulate; int2 packed cache",
        "data": "synthetic (seeded N(0,1) Q/K/V drawn on the device, with "
                "attention sink, planted heavy hitters and key outlier "
                "channels)",
        "config": rec["config"],
    }
    for key in ("decode_pct_hbm_peak", "prefill_tflops",
                "prefill_pct_mfma_fp16_peak", "phase_ms_per_step", "roofline",
                "roofline_prefill", "decode_mass_audit", "input_generation_s"):
        result[key] = rec[key]
    if not args.no_persistence:
        result["persistence_audit"] = persistence_audit(st)
        log("persistence audit done")
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(st, args.cpu_seconds)
        log("cpu baseline done")
    del st
    torch.cuda.empty_cache()
    subs = {}
    for cid in [int(x) for x in args.sub_configs.split(",") if x.strip()]:
        sub, st = run_workload(cid, args.sub_steps, 1, args, stream,
                               headline=False)
        del st
        torch.cuda.empty_cache()
        subs[sub["workload"]] = sub
    if subs:
        result["sub_records"] = subs
    if not args.no_mixed:
        mixed = {}
        for cid in [int(x) for x in args.mixed_configs.split(",") if x.strip()]:
            from bit_quantized_attention_two_amd import configs
            mixed[configs.get(cid)["name"]] = mixed_records(stream, cid)
            torch.cuda.empty_cache()
            log("mixed-precision records of workload %d done" % cid)
        result["mixed_precision"] = mixed
    if not args.no_fused_tail:
        result["fused_prefill_tail"] = [fused_tail_record(stream, cid)
                                        for cid in (2, 4, 5)]
        log("fused prefill tail records done")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
