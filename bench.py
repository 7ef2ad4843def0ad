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
Inputs (prompt Q/K/V of every layer and the decode-step q/k/v) are resident
in HBM before the timed region.

Printed: one JSON line.  `value` is the decode phase's algorithmic bytes
(packed codes + fp16 scale/zero + fp16 residual + q/o, counted as the method
must move them) divided by the decode phase's wall time; the prefill phase's
algorithmic TFLOP/s (3 D n (n+1) per query head and layer: QK^T and PV of
pass 1, QK^T again in pass 2) is reported next to it.  `roofline` is for the
decode-attention call, timed with HIP events on the stream it runs on.
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.
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


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=3)
    p.add_argument("--warmup", type=int, default=1)
    p.add_argument("--config", type=int, default=2,
                   help="workload id (configs.py); default: the 4096-token "
                        "Llama2-7B-shaped stack")
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
                        "workload N (two alternating caches) and print it; "
                        "the workload for the decode kernels' counters")
    p.add_argument("--no-persistence", action="store_true",
                   help="skip the persistence audit (re-selection every 32 "
                        "decode steps, overlap with the prefill heavy "
                        "hitters)")
    p.add_argument("--no-large-decode", action="store_true",
                   help="skip the decode-call timing at the 13B-shaped "
                        "batched layer (16 x 40 kv heads, 4096 packed tokens)")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="rough CPU budget of the oracle baseline")
    p.add_argument("--traffic-probe", action="store_true",
                   help="run only the short workload whose HBM counters "
                        "(rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE) give the "
                        "roofline's traffic: a 256 MiB device copy for "
                        "calibration, then one decode call per layer at the "
                        "end-of-step cache state")
    return p.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_llama2_7b_4k_traffic.md")
DECODE_SRC = os.path.join(ROOT, "bit_quantized_attention_two_amd", "csrc",
                          "decode.hip")


def measured_traffic(config_id):
    """HBM bytes per decode call from the committed counter summary, or None
    when it does not cover this workload or the decode source has changed
    since the counters were taken."""
    import hashlib
    if config_id != 2 or not os.path.exists(TRAFFIC_FILE):
        return None
    fields = {}
    for line in open(TRAFFIC_FILE):
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


def traffic_probe():
    """Workload for the traffic counters (see --traffic-probe)."""
    import torch
    from bit_quantized_attention_two_amd import configs, minikv
    c = configs.get(2)
    B, Hq, Hkv, D, n, L = c["B"], c["Hq"], c["Hkv"], c["D"], c["n"], c["L"]
    ks, r = minikv.pyramid_budgets(n, L, c["hh"], c["rw"], c["depth"],
                                   c["pyramid"])
    dims = minikv.make_dims(B, Hq, Hkv, D, c["Gk"], c["Gv"], c["residual_cap"])
    torch.manual_seed(0)
    src = torch.randn(64 * 1024 * 1024, device="cuda")      # 256 MiB
    dst = torch.empty_like(src)
    k = torch.randn(B, Hkv, n, D, device="cuda").half()
    v = torch.randn(B, Hkv, n, D, device="cuda").half()
    kn = torch.randn(B, Hkv, D, device="cuda").half()
    caches = []
    for l in range(L):
        m = ks[l] + r
        sel = (torch.arange(m, device="cuda", dtype=torch.int64) * n // m
               ).int().repeat(B, Hkv, 1).contiguous()
        cache = minikv.LayerCache(dims, (m // 16) * 16 + 256)
        minikv.pack(dims, k, v, sel, cache)
        for _ in range(c["decode_steps"]):          # end-of-step state
            minikv.append(dims, cache, kn, kn)
        caches.append(cache)
    q = torch.randn(B, Hq, D, device="cuda").half()
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
    print(json.dumps({"copy_bytes": src.numel() * 4, "decode_calls": L,
                      "algorithmic_bytes_per_call": alg / L}), flush=True)


def layer_decode_roofline(stream, config_id=3):
    """Decode-attention call at one layer of a workload, in its bandwidth
    regime: layer 0's selection (its heavy-hitter budget plus the recent
    window) packed, then enough decode-step tokens appended to hold 64 in
    the fp16 residual.  At the Llama2-13B-shaped batched layer (batch 16, 40
    kv heads, D 128) that is 4096 packed + 64 residual tokens per kv head,
    ~360 MB per call; the bench workload's 4096-token layer (~9 MB per call)
    is latency-bound instead.  Two such caches alternate (more than the
    256 MB last-level cache at the 13B shape, so no call finds the previous
    call's data there), timed as a graph of back-to-back calls between HIP
    events on `stream`: 10 replays to warm up (the GPU's clock ramps up
    under sustained load; single replays right after other work run ~15%
    slower), then the median of 10 replays."""
    import torch
    from bit_quantized_attention_two_amd import configs, minikv
    c = configs.get(config_id)
    B, Hq, Hkv, D, n, L = c["B"], c["Hq"], c["Hkv"], c["D"], c["n"], c["L"]
    dims = minikv.make_dims(B, Hq, Hkv, D, c["Gk"], c["Gv"], c["residual_cap"])
    ks, r = minikv.pyramid_budgets(n, L, c["hh"], c["rw"], c["depth"],
                                   c["pyramid"])
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
        assert cache.n_res == res
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
    for _ in range(10):                          # the clock ramps up under
        gr.replay()                              # sustained load: warm up
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


def persistence_audit(config_id, layer=0, every=32):
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
    from bit_quantized_attention_two_amd import configs, minikv, synth
    c = configs.get(config_id)
    B, Hq, Hkv, D, n, L = c["B"], c["Hq"], c["Hkv"], c["D"], c["n"], c["L"]
    S = c["decode_steps"]
    ks, r = minikv.pyramid_budgets(n, L, c["hh"], c["rw"], c["depth"],
                                   c["pyramid"])
    n_hh = int(ks[layer])
    dims = minikv.make_dims(B, Hq, Hkv, D, c["Gk"], c["Gv"], c["residual_cap"])
    q, k, v = synth.gen_prefill(config_id, layer)
    steps = [synth.gen_decode_step(config_id, layer, t, B, Hq, Hkv, D)
             for t in range(S)]
    ext = [np.concatenate([x, np.stack([st[i] for st in steps], axis=2)],
                          axis=2) for i, x in enumerate((q, k, v))]
    Q, K, V = (torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in ext)
    points = list(range(0, S + 1, every))
    if points[-1] != S:
        points.append(S)
    hh0, rows, ms = None, [], 0.0
    for t in points:
        sub = [x[:, :, :n + t].contiguous() for x in (Q, K, V)]
        a, b = (torch.cuda.Event(enable_timing=True) for _ in range(2))
        a.record()
        _, _, sel = minikv.prefill_select(dims, *sub, n_hh, r + t)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        hh = sel[..., :n_hh].cpu().numpy().reshape(B * Hkv, n_hh)
        if hh0 is None:
            hh0 = hh
        ov = np.array([np.intersect1d(x, y).size for x, y in zip(hh, hh0)]) / n_hh
        rows.append((t, float(ov.mean()), float(ov.min())))
    return {"layer": layer, "heavy_hitters": n_hh, "recent": r,
            "steps": [x[0] for x in rows],
            "overlap_mean": [round(x[1], 4) for x in rows],
            "overlap_min": [round(x[2], 4) for x in rows],
            "reselect_ms_at_last_step": round(ms, 3)}


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


def main():
    args = parse()
    if args.traffic_probe:
        traffic_probe()
        return
    if args.decode_probe:
        import torch
        print(json.dumps(layer_decode_roofline(torch.cuda.current_stream(),
                                               args.decode_probe)), flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU "
              "path (each GPU would run the same kernels on its own share of "
              "kv heads, with no exchange); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from bit_quantized_attention_two_amd import configs, minikv, synth
    minikv.lib()
    assert torch.cuda.is_available(), "needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    c = configs.get(args.config)
    B, Hq, Hkv, D, n, L = c["B"], c["Hq"], c["Hkv"], c["D"], c["n"], c["L"]
    Gk, Gv, nr, S = c["Gk"], c["Gv"], c["residual_cap"], c["decode_steps"]
    ks, r = minikv.pyramid_budgets(n, L, c["hh"], c["rw"], c["depth"],
                                   c["pyramid"])
    dims = minikv.make_dims(B, Hq, Hkv, D, Gk, Gv, nr)
    nl = args.distinct_layers or L
    ns = args.distinct_steps or S

    t0 = time.time()
    qkv = [None] * nl
    import concurrent.futures as cf
    with cf.ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        futs = {ex.submit(synth.gen_prefill, args.config, l): l
                for l in range(nl)}
        for f in cf.as_completed(futs):
            qkv[futs[f]] = tuple(torch.from_numpy(a).to(dev) for a in f.result())
    dq = torch.empty((ns, nl, B, Hq, D), dtype=torch.float16, device=dev)
    dk = torch.empty((ns, nl, B, Hkv, D), dtype=torch.float16, device=dev)
    dv = torch.empty_like(dk)
    for s in range(ns):
        for l in range(nl):
            a, b_, c_ = synth.gen_decode_step(args.config, l, s, B, Hq, Hkv, D)
            dq[s, l].copy_(torch.from_numpy(a))
            dk[s, l].copy_(torch.from_numpy(b_))
            dv[s, l].copy_(torch.from_numpy(c_))
    gen_s = time.time() - t0

    outs, caches, sels, cols = [], [], [], []
    ws_pref = torch.empty(minikv.prefill_ws_bytes(dims, n), dtype=torch.uint8,
                          device=dev)
    for l in range(L):
        m = ks[l] + r
        cap = ((m // Gk) * Gk + S + nr + Gk - 1) // Gk * Gk
        caches.append(minikv.LayerCache(dims, cap, dev))
        outs.append(torch.empty((B, Hq, n, D), dtype=torch.float16, device=dev))
        cols.append(torch.empty((B, Hkv, n), dtype=torch.float32, device=dev))
        sels.append(torch.empty((B, Hkv, m), dtype=torch.int32, device=dev))
    max_cap = max(x.capacity for x in caches)
    ws_dec = torch.zeros(minikv.decode_ws_bytes(dims, max_cap),
                         dtype=torch.uint8, device=dev)
    od = torch.empty((B, Hq, D), dtype=torch.float16, device=dev)
    stream = torch.cuda.current_stream()

    # One step in model order.  The prefill part runs every layer's
    # prefill+select and pack; the decode part runs, for every decode step,
    # every layer's append and decode attention.
    dec_bytes_per_call = []

    def prefill_part():
        for l in range(L):
            q, k, v = qkv[l % nl]
            minikv.prefill_select(dims, q, k, v, ks[l], r, o=outs[l],
                                  col=cols[l], sel=sels[l], ws=ws_pref)
            minikv.pack(dims, k, v, sels[l], caches[l])

    def decode_part():
        dec_bytes_per_call.clear()
        for s in range(S):
            for l in range(L):
                cache = caches[l]
                # append + decode attention, fused unless the residual flushes
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

    # warm-up (eager), then capture one step as two graphs
    for _ in range(max(1, args.warmup)):
        prefill_part()
        decode_part()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    graphs = None
    if not args.eager:
        side.wait_stream(stream)
        graphs = (capture(prefill_part, side), capture(decode_part, side))
        stream.wait_stream(side)
        for _ in range(args.warmup):
            graphs[0].replay()
            graphs[1].replay()
        torch.cuda.synchronize()

    phase = []
    t_start = time.perf_counter()
    for _ in range(args.steps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e2 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        graphs[0].replay() if graphs else prefill_part()
        e1.record(stream)
        graphs[1].replay() if graphs else decode_part()
        e2.record(stream)
        phase.append((e0, e1, e2, sum(dec_bytes_per_call)))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start

    # Per-call durations of the two dominant calls, measured right after the
    # timed steps on the same stream with HIP events: the decode-attention
    # call of every layer, in its end-of-step cache state, replayed
    # back-to-back from a graph (R rounds of all layers), and each layer's
    # prefill+select call between its own events.
    R = 8
    side.wait_stream(stream)
    g_kern = capture(lambda: [minikv.decode_attn(dims, caches[l],
                                                 dq[0, l % nl], o=od,
                                                 ws=ws_dec)
                              for _ in range(R) for l in range(L)], side)
    stream.wait_stream(side)
    g_kern.replay()
    ka, kb = (torch.cuda.Event(enable_timing=True) for _ in range(2))
    ka.record(stream)
    g_kern.replay()
    kb.record(stream)
    torch.cuda.synchronize()
    dec_call_ms = np.array([ka.elapsed_time(kb) / (R * L)])
    # the same calls with the persistence audit's per-token mass output
    mass = torch.zeros((B, Hkv, max_cap + nr), dtype=torch.float32,
                       device=dev)
    ws_mass = torch.empty(minikv.decode_mass_ws_bytes(dims, max_cap),
                          dtype=torch.uint8, device=dev)
    side.wait_stream(stream)
    g_mass = capture(lambda: [minikv.decode_attn_mass(dims, caches[l],
                                                      dq[0, l % nl], mass,
                                                      o=od, ws=ws_mass)
                              for _ in range(R) for l in range(L)], side)
    stream.wait_stream(side)
    g_mass.replay()
    ka.record(stream)
    g_mass.replay()
    kb.record(stream)
    torch.cuda.synchronize()
    mass_call_ms = ka.elapsed_time(kb) / (R * L)
    dec_call_bytes = np.array([decode_bytes(c, x.n_packed, x.n_res)
                               for x in caches], np.float64)
    # each layer's call on its own (a graph of R back-to-back calls of that
    # layer between HIP events): the per-layer median and p90
    layer_us = []
    for l in range(L):
        side.wait_stream(stream)
        g_l = capture(lambda: [minikv.decode_attn(dims, caches[l],
                                                  dq[0, l % nl], o=od,
                                                  ws=ws_dec)
                               for _ in range(R)], side)
        stream.wait_stream(side)
        g_l.replay()
        ka.record(stream)
        g_l.replay()
        kb.record(stream)
        torch.cuda.synchronize()
        layer_us.append(ka.elapsed_time(kb) * 1e3 / R)
        del g_l
    pre_call_ms = []
    for l in range(L):
        q, k, v = qkv[l % nl]
        a, b = (torch.cuda.Event(enable_timing=True) for _ in range(2))
        a.record(stream)
        minikv.prefill_select(dims, q, k, v, ks[l], r, o=outs[l], col=cols[l],
                              sel=sels[l], ws=ws_pref)
        b.record(stream)
        pre_call_ms.append((a, b))
    torch.cuda.synchronize()
    pre_call_ms = [a.elapsed_time(b) for a, b in pre_call_ms]

    pre_ms = sum(e0.elapsed_time(e1) for e0, e1, _, _ in phase)
    dec_ms = sum(e1.elapsed_time(e2) for _, e1, e2, _ in phase)
    dec_bytes = sum(x[3] for x in phase)
    value = dec_bytes / (dec_ms * 1e-3) / 1e9
    pre_tflops = prefill_flops(c) * L * args.steps / (pre_ms * 1e-3) / 1e12
    ms_per_step = wall * 1e3 / args.steps

    avg_dec_ms = float(dec_call_ms.mean())
    avg_dec_bytes = float(dec_call_bytes.mean())
    achieved = avg_dec_bytes / (avg_dec_ms * 1e-3) / 1e9
    pre_call_ms = np.array(pre_call_ms)
    pre_achieved = prefill_flops(c) / (pre_call_ms.mean() * 1e-3) / 1e12

    result = {
        "metric": "packed-KV decode attention GB/s (% HBM peak) + prefill "
                  "selective-attn TFLOP/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 in, fp32 accumulate; int2 packed cache",
        "data": "synthetic (seeded N(0,1) Q/K/V with attention sink, planted "
                "heavy hitters and key outlier channels)",
        "config": {
            "workload": c["name"], "config_id": args.config, "batch": B,
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
        "decode_pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "prefill_tflops": round(pre_tflops, 2),
        "prefill_pct_mfma_fp16_peak": round(100 * pre_tflops /
                                            MFMA_FP16_PEAK_TFLOPS, 2),
        "phase_ms_per_step": {"prefill": round(pre_ms / args.steps, 3),
                              "decode": round(dec_ms / args.steps, 3)},
        "roofline": {
            "kernel": "minikv_decode_attn (split-KV decode + combine "
                      "kernels), all layers, end-of-step cache state",
            "bound": "hbm", "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(args.config),
            "avg_launch_us": round(avg_dec_ms * 1e3, 3),
            "algorithmic_bytes_per_launch": int(avg_dec_bytes),
            "launches": R * L,
            "per_layer_call_us": {"median": round(float(np.median(layer_us)), 3),
                                  "p90": round(float(np.percentile(layer_us, 90)), 3),
                                  "min": round(min(layer_us), 3),
                                  "max": round(max(layer_us), 3)},
        },
        "roofline_prefill": {
            "kernel": "minikv_prefill_select (pass 1 + pass 2 + select)",
            "bound": "mfma", "achieved": round(pre_achieved, 2),
            "peak": MFMA_FP16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(pre_achieved / MFMA_FP16_PEAK_TFLOPS, 4),
            "avg_launch_us": round(float(pre_call_ms.mean()) * 1e3, 3),
            "algorithmic_flops_per_launch": prefill_flops(c),
        },
        "decode_mass_audit": {
            "kernel": "minikv_decode_attn_mass (decode + per-token "
                      "attention mass, accumulated)",
            "avg_launch_us": round(mass_call_ms * 1e3, 3),
            "vs_decode_call": round(mass_call_ms / avg_dec_ms, 3),
        },
        "input_generation_s": round(gen_s, 1),
    }
    if not args.no_persistence:
        result["persistence_audit"] = persistence_audit(args.config)
    if not args.no_large_decode:
        del qkv, outs, cols, graphs, g_kern, g_mass
        torch.cuda.empty_cache()
        result["roofline_decode_large"] = layer_decode_roofline(stream, 3)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, c, ks, r, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def cpu_baseline(args, c, ks, r, budget_s):
    """The oracle, as it is, on host threads: decode attention of sampled
    units of layer 0 (packed by the oracle itself from the same seeded
    inputs), reported in the metric's unit, plus the oracle's prefill rate on
    one unit for context."""
    import concurrent.futures as cf

    import oracle
    from bit_quantized_attention_two_amd import synth
    oracle.build(force=False)
    cores = min(16, os.cpu_count() or 1)
    B, Hq, Hkv, D, n = c["B"], c["Hq"], c["Hkv"], c["D"], c["n"]
    g = Hq // Hkv
    m = ks[0] + r
    q, k, v = synth.gen_prefill(args.config, 0, batches=[0])
    units = [(0, h) for h in range(Hkv)]
    cap = ((m // c["Gk"]) * c["Gk"] + 256)
    oc = oracle.OracleCache(1, Hkv, D, c["Gk"], c["Gv"], cap,
                            c["residual_cap"])
    # heavy hitters: the oracle's own prefill scores would cost O(n^2) per
    # unit; use its selection on the first unit's scores for every unit
    t0 = time.perf_counter()
    _, _, col = oracle.prefill_unit(q[0, :g], k[0, 0], v[0, 0])
    t_pref = time.perf_counter() - t0
    sel0 = oracle.select(col, ks[0], r)
    sel = np.tile(sel0, (1, Hkv, 1))
    t0 = time.perf_counter()
    oc.pack(k, v, sel, workers=cores)
    t_pack = time.perf_counter() - t0
    qd, _, _ = synth.gen_decode_step(args.config, 0, 0, 1, Hq, Hkv, D)
    nbytes_call = decode_bytes(dict(c, B=1), oc.n_packed, oc.n_res)
    reps = 0
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(cores) as ex:
        while True:
            list(ex.map(lambda u: oc.decode_unit(qd[0, u[1] * g:(u[1] + 1) * g],
                                                 0, u[1]), units))
            reps += 1
            if time.perf_counter() - t0 > budget_s / 2 or reps >= 10000:
                break
    t_dec = time.perf_counter() - t0
    return {
        "value": round(nbytes_call * reps / t_dec / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": "decode attention of all %d kv-head units of layer 0, batch "
                  "element 0 (%d packed + %d residual tokens each), repeated "
                  "%d times on %d threads; fp64 oracle" %
                  (Hkv, oc.n_packed, oc.n_res, reps, cores),
        "prefill_tflops_one_unit_one_thread": round(
            prefill_flops(dict(c, B=1, Hq=g)) / t_pref / 1e12, 6),
        "pack_s_all_units": round(t_pack, 3),
        "seconds": round(t_dec + t_pref + t_pack, 2),
    }


if __name__ == "__main__":
    main()
