"""Seeded synthetic inputs, shared by the tests, the benchmark and the smoke
check.  This module holds no arithmetic of the method itself: it only draws
random tensors with the structure the MiniKV pages describe (an attention
sink, a few heavy-hitter keys aligned with the queries, and a handful of key
channels with large outliers -- Pith review of MiniKV, Fig. 10 caption on the
attention distribution, and the verdict record's supporting citation on
channel outliers in keys).

Every draw uses numpy's PCG64 seeded with a tuple
(SEED, config, layer, tag, index) so that any batch element or decode step can
be regenerated on its own.  Tags: 0 Q, 1 K, 2 V, 3 outlier channels,
4 heavy-hitter positions, 5/6/7 decode q/k/v, 8 score vectors, 9 selections.
All tensors are produced in fp32 and rounded once to fp16 (numpy astype, RNE).
"""
import numpy as np

from . import configs

SINK_GAIN = 8.0       # sink key = SINK_GAIN * sqrt(D) * u
HH_GAIN = 4.0         # planted heavy hitters = HH_GAIN * sqrt(D) * u
N_HH_PLANTED = 8
N_OUTLIER_CH = 4
OUTLIER_GAIN = 10.0


def rng(*key):
    return np.random.default_rng([configs.SEED] + [int(x) for x in key])


def outlier_channels(cfg_id, layer, Hkv, D):
    """[Hkv][N_OUTLIER_CH] distinct key channels per kv head."""
    r = rng(cfg_id, layer, 3)
    nch = min(N_OUTLIER_CH, D)
    return np.stack([np.sort(r.choice(D, nch, replace=False))
                     for _ in range(Hkv)])


def gen_unit_batch(cfg_id, layer, b, Hq, Hkv, n, D, r_window,
                   structure=True):
    """Q [Hq][n][D], K, V [Hkv][n][D] (fp16) for batch element b."""
    g = Hq // Hkv
    q = rng(cfg_id, layer, 0, b).standard_normal((Hq, n, D), np.float32)
    k = rng(cfg_id, layer, 1, b).standard_normal((Hkv, n, D), np.float32)
    v = rng(cfg_id, layer, 2, b).standard_normal((Hkv, n, D), np.float32)
    if structure and n > 0:
        hr = rng(cfg_id, layer, 4, b)
        och = outlier_channels(cfg_id, layer, Hkv, D)
        for h in range(Hkv):
            u = q[h * g:(h + 1) * g].mean(axis=(0, 1), dtype=np.float64)
            nu = np.linalg.norm(u)
            u = (u / nu if nu > 0 else np.ones(D) / np.sqrt(D)).astype(np.float32)
            k[h, 0] = SINK_GAIN * np.sqrt(D) * u
            hi = max(n - r_window, 1)
            cnt = min(N_HH_PLANTED, hi - 1)
            if cnt > 0:
                pos = hr.choice(np.arange(1, hi), cnt, replace=False)
                k[h, pos] = HH_GAIN * np.sqrt(D) * u
            k[h][:, och[h]] *= OUTLIER_GAIN
    return q.astype(np.float16), k.astype(np.float16), v.astype(np.float16)


def gen_prefill(cfg_id, layer, batches=None, structure=True, c=None):
    """Q [nb][Hq][n][D], K, V [nb][Hkv][n][D] fp16 for the listed batches."""
    c = c or configs.get(cfg_id)
    batches = range(c["B"]) if batches is None else batches
    r_window = c["n"] * c["rw"][0] // c["rw"][1]
    parts = [gen_unit_batch(cfg_id, layer, b, c["Hq"], c["Hkv"], c["n"],
                            c["D"], r_window, structure) for b in batches]
    return tuple(np.stack(x) for x in zip(*parts))


def gen_decode_step(cfg_id, layer, step, B, Hq, Hkv, D, structure=True):
    """q [B][Hq][D], k, v [B][Hkv][D] fp16 for one decode step."""
    q = rng(cfg_id, layer, 5, step).standard_normal((B, Hq, D), np.float32)
    k = rng(cfg_id, layer, 6, step).standard_normal((B, Hkv, D), np.float32)
    v = rng(cfg_id, layer, 7, step).standard_normal((B, Hkv, D), np.float32)
    if structure:
        och = outlier_channels(cfg_id, layer, Hkv, D)
        for h in range(Hkv):
            k[:, h][:, och[h]] *= OUTLIER_GAIN
    return q.astype(np.float16), k.astype(np.float16), v.astype(np.float16)


def gen_scores(seed, units, n, kind="random"):
    """fp32 cumulative-score-like vectors [units][n] for selection tests.

    kind: "random" (distinct-ish positive values), "ties" (values from a set
    of 7 levels, so ties are everywhere), "const" (all equal),
    "decreasing" (strictly decreasing in the index).
    """
    r = rng(8, seed)
    if kind == "random":
        x = r.exponential(1.0, (units, n)).astype(np.float32)
    elif kind == "ties":
        x = r.integers(0, 7, (units, n)).astype(np.float32) * 0.25
    elif kind == "const":
        x = np.full((units, n), 1.5, np.float32)
    elif kind == "decreasing":
        x = np.tile(np.linspace(1000.0, 1.0, n, dtype=np.float32), (units, 1))
    else:
        raise ValueError(kind)
    return np.ascontiguousarray(x)


def gen_selection(seed, units, n, m):
    """Random ascending index sets [units][m] drawn from [0, n)."""
    r = rng(9, seed)
    return np.stack([np.sort(r.choice(n, m, replace=False)).astype(np.int32)
                     for _ in range(units)])


def gen_kv(seed, units, n, D, outliers=True):
    """Plain fp16 K, V [units][n][D] for codec tests (N(0,1), a few key
    channels scaled by OUTLIER_GAIN)."""
    r = rng(10, seed)
    k = r.standard_normal((units, n, D), np.float32)
    v = r.standard_normal((units, n, D), np.float32)
    if outliers:
        for u in range(units):
            ch = r.choice(D, min(N_OUTLIER_CH, D), replace=False)
            k[u][:, ch] *= OUTLIER_GAIN
    return k.astype(np.float16), v.astype(np.float16)


# ------------------------------------------------ device-side generation --
# The benchmark's full-size workloads (up to 51 GB of prompt tensors) are
# drawn on the GPU with torch's counter-based generator instead of numpy's
# PCG64, with the same recipe: N(0,1) fp32 draws, the sink and heavy-hitter
# keys along the normalised mean query of the kv head's group, the same
# outlier channels (numpy, tag 3) and planted positions (numpy, tag 4), and
# one rounding to fp16.  Values differ from gen_prefill's; the structure and
# distributions are the same.

def _torch_gen(device, *key):
    import torch
    seed = int(rng(*key).integers(0, 2 ** 62))
    return torch.Generator(device=device).manual_seed(seed)


def gen_prefill_device(cfg_id, layer, device, c=None, structure=True):
    """Q [B][Hq][n][D], K, V [B][Hkv][n][D] fp16 tensors on `device`."""
    import torch
    c = c or configs.get(cfg_id)
    B, Hq, Hkv, n, D = c["B"], c["Hq"], c["Hkv"], c["n"], c["D"]
    g = Hq // Hkv
    r_window = n * c["rw"][0] // c["rw"][1]
    q = torch.empty((B, Hq, n, D), dtype=torch.float16, device=device)
    k = torch.empty((B, Hkv, n, D), dtype=torch.float16, device=device)
    v = torch.empty_like(k)
    och = outlier_channels(cfg_id, layer, Hkv, D)
    for b in range(B):
        gq = _torch_gen(device, cfg_id, layer, 0, b)
        gk = _torch_gen(device, cfg_id, layer, 1, b)
        gv = _torch_gen(device, cfg_id, layer, 2, b)
        hr = rng(cfg_id, layer, 4, b)
        for h in range(Hkv):
            qf = torch.randn((g, n, D), generator=gq, device=device)
            kf = torch.randn((n, D), generator=gk, device=device)
            v[b, h] = torch.randn((n, D), generator=gv, device=device).half()
            if structure and n > 0:
                u = qf.double().mean(dim=(0, 1))
                nu = torch.linalg.norm(u)
                u = (u / nu if nu > 0 else
                     torch.full((D,), D ** -0.5, dtype=torch.float64,
                                device=device)).float()
                kf[0] = SINK_GAIN * np.sqrt(D) * u
                hi = max(n - r_window, 1)
                cnt = min(N_HH_PLANTED, hi - 1)
                if cnt > 0:
                    pos = hr.choice(np.arange(1, hi), cnt, replace=False)
                    kf[torch.from_numpy(pos).to(device)] = HH_GAIN * np.sqrt(D) * u
                kf[:, torch.from_numpy(och[h]).to(device)] *= OUTLIER_GAIN
            q[b, h * g:(h + 1) * g] = qf.half()
            k[b, h] = kf.half()
    return q, k, v


def gen_decode_device(cfg_id, steps, layers, device, c=None):
    """q [steps][layers][B][Hq][D], k, v [steps][layers][B][Hkv][D] fp16 on
    `device`: N(0,1) draws with the layer's key outlier channels."""
    import torch
    c = c or configs.get(cfg_id)
    B, Hq, Hkv, D = c["B"], c["Hq"], c["Hkv"], c["D"]
    q = torch.empty((steps, layers, B, Hq, D), dtype=torch.float16, device=device)
    k = torch.empty((steps, layers, B, Hkv, D), dtype=torch.float16, device=device)
    v = torch.empty_like(k)
    for l in range(layers):
        gen = _torch_gen(device, cfg_id, l, 5, 0)
        q[:, l] = torch.randn((steps, B, Hq, D), generator=gen, device=device).half()
        kf = torch.randn((steps, B, Hkv, D), generator=gen, device=device)
        och = outlier_channels(cfg_id, l, Hkv, D)
        for h in range(Hkv):
            kf[:, :, h][:, :, torch.from_numpy(och[h]).to(device)] *= OUTLIER_GAIN
        k[:, l] = kf.half()
        v[:, l] = torch.randn((steps, B, Hkv, D), generator=gen, device=device).half()
    return q, k, v
