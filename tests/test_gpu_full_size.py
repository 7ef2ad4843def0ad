"""End to end at the full sizes of the three large workloads (Llama2-13B-
shaped batch 16 x 40 heads x 8192 tokens; Mistral-7B-shaped GQA batch 4 x
32768; Llama-3-8B-shaped GQA 131072 tokens), layers 0 and L-1, each exactly
as the bench runs it: one minikv_prefill_select call over all units, pack of
the GPU's own selection, then minikv_append_decode steps crossing a residual
flush (at the 131072-token workload: its 64 decode steps, no flush).

Checked against the oracle:
  - every unit: sum_j col_j = g n (rows of a softmax sum to one), and the
    selection protocol's part 1 (the oracle's selection over the GPU's own
    scores is the GPU's selection);
  - the golden units (layer 0; tests/golden/make_golden_scores.py, oracle
    only): every column of col element-wise, and part 2 of the protocol
    (only boundary swaps against the oracle's own selection);
  - O and LSE of sampled query rows (plus the last 64) of two units;
  - the packed cache bit for bit on sampled units (the oracle's pack of the
    GPU's selection, then its appends and flush), and the decode outputs of
    those units at the first, the flushing and the last step."""
import concurrent.futures as cf
import os

import numpy as np
import pytest

import oracle
from bit_quantized_attention_two_amd import configs, synth
from gpu_util import (assert_close, cache_to_numpy, check_selection, dev16,
                      lib_budgets, require_gpu, say)

pytestmark = pytest.mark.gpu

WORKERS = min(16, os.cpu_count() or 1)
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
PACKED = (("kq", "kq"), ("k_scale", "ks"), ("k_zero", "kz"), ("vq", "vq"),
          ("v_scale", "vs"), ("v_zero", "vz"))


def _golden(c, layer, b, h):
    path = os.path.join(GOLDEN, "scores_%s_l%d_b%d_h%d.npy" % (
        c["name"].replace("-", "_"), layer, b, h))
    return np.load(path) if os.path.exists(path) else None


@pytest.mark.parametrize("cfg_id,layer", [(3, 0), (3, 39), (4, 0), (4, 31),
                                          (5, 0), (5, 31)])
def test_full_size_pipeline(cfg_id, layer):
    torch, mk = require_gpu()
    c = configs.get(cfg_id)
    B, Hq, Hkv, D, n, g = c["B"], c["Hq"], c["Hkv"], c["D"], c["n"], c["g"]
    Gk, Gv, nr = c["Gk"], c["Gv"], c["residual_cap"]
    ks, r = lib_budgets(mk, c)
    n_hh = int(ks[layer])
    m = n_hh + r
    steps = min(c["decode_steps"], nr)
    say("full-size generate", dict(cfg=cfg_id, layer=layer, B=B, n=n))
    q, k, v = synth.gen_prefill(cfg_id, layer)
    dims = mk.make_dims(B, Hq, Hkv, D, Gk, Gv, nr)
    kd, vd = dev16(torch, k), dev16(torch, v)
    lse = torch.empty((B, Hq, n), dtype=torch.float32, device="cuda")
    say("full-size prefill_select", dict(cfg=cfg_id, layer=layer, n_hh=n_hh, r=r))
    o, col, sel = mk.prefill_select(dims, dev16(torch, q), kd, vd, n_hh, r,
                                    lse=lse)
    cap = ((m // Gk) * Gk + steps + nr + Gk - 1) // Gk * Gk
    cache = mk.LayerCache(dims, cap)
    mk.pack(dims, kd, vd, sel, cache)
    col_h, sel_h = col.cpu().numpy(), sel.cpu().numpy()

    # every unit: rows sum to one; selection part 1
    np.testing.assert_allclose(col_h.sum(-1), g * n, rtol=1e-4)
    units = [(b, h) for b in range(B) for h in range(Hkv)]
    for b, h in units:
        check_selection(sel_h[b, h], col_h[b, h], None, None, n_hh, r)

    # golden units: every column, and part 2
    golden = [(b, h) for b, h in units if _golden(c, layer, b, h) is not None]
    if layer == 0:
        assert golden, "no golden scores for %s layer 0" % c["name"]
    swaps = 0
    for b, h in golden:
        ref = _golden(c, layer, b, h)
        assert_close(col_h[b, h], ref, "col b%d h%d (every column)" % (b, h))
        swaps += check_selection(sel_h[b, h], col_h[b, h],
                                 oracle.select(ref, n_hh, r), ref, n_hh, r)
    print("golden units %s, boundary swaps %d" % (golden, swaps), flush=True)

    # O and LSE on sampled rows of two units
    rr = np.random.default_rng(1000 * cfg_id + layer)
    rows = np.unique(np.concatenate([rr.choice(n - 64, 24, replace=False),
                                     np.arange(n - 64, n)])).astype(np.int32)
    two = [units[0], units[-1]]
    say("full-size oracle rows", dict(cfg=cfg_id, layer=layer, units=two))
    o_h, lse_h = o.cpu().numpy(), lse.cpu().numpy()
    del o
    with cf.ThreadPoolExecutor(WORKERS) as ex:
        refs = list(ex.map(lambda u: oracle.prefill_rows(
            q[u[0], u[1] * g:(u[1] + 1) * g], k[u[0], u[1]], v[u[0], u[1]],
            rows[u[2]::WORKERS // 2 or 1], want_col=False),
            [(b, h, s) for b, h in two for s in range(WORKERS // 2 or 1)]))
    per = WORKERS // 2 or 1
    for i, (b, h) in enumerate(two):
        for s in range(per):
            ro, rl, _ = refs[i * per + s]
            rs = rows[s::per]
            assert_close(o_h[b, h * g:(h + 1) * g][:, rs], ro, "O b%d h%d" % (b, h))
            assert_close(lse_h[b, h * g:(h + 1) * g][:, rs], rl, "LSE b%d h%d" % (b, h))
    del o_h, lse_h

    # pack bit for bit on sampled units, then appends (one flush) and decode
    sample = sorted(set(golden) | {units[0], units[-1], units[len(units) // 2]})
    oc = oracle.OracleCache(B, Hkv, D, Gk, Gv, cap, nr)
    oc.pack(k, v, sel_h, units=sample, workers=WORKERS)
    del q
    torch.cuda.synchronize()

    def compare_bits(when):
        gc = cache_to_numpy(cache)
        for b, h in sample:
            u = b * Hkv + h
            for gname, oname in PACKED:
                assert np.array_equal(gc[gname][u], getattr(oc, oname)[b, h]), \
                    (when, gname, b, h)
            assert np.array_equal(gc["k_res"][u][:oc.n_res], oc.kres[b, h][:oc.n_res])
            assert np.array_equal(gc["v_res"][u][:oc.n_res], oc.vres[b, h][:oc.n_res])

    compare_bits("after pack")
    ws = torch.zeros(mk.decode_ws_bytes(dims, cap), dtype=torch.uint8,
                     device="cuda")
    flushed_at = None
    for s in range(steps):
        qs, kn, vn = synth.gen_decode_step(cfg_id, layer, s, B, Hq, Hkv, D)
        od = mk.append_decode(dims, cache, dev16(torch, kn), dev16(torch, vn),
                              dev16(torch, qs), ws=ws)
        oc.append(kn, vn)
        if oc.n_res == 0:
            flushed_at = s
        if s in (0, steps - 1) or s == flushed_at:
            say("full-size decode", dict(cfg=cfg_id, layer=layer, step=s))
            od = od.cpu().numpy()
            compare_bits("step %d" % s)
            with cf.ThreadPoolExecutor(WORKERS) as ex:
                refs = list(ex.map(lambda u: oc.decode_unit(
                    qs[u[0], u[1] * g:(u[1] + 1) * g], u[0], u[1]), sample))
            for (b, h), ref in zip(sample, refs):
                assert_close(od[b, h * g:(h + 1) * g], ref,
                             "decode b%d h%d step %d" % (b, h, s))
    assert cache.n_packed == oc.n_packed and cache.n_res == oc.n_res
    if steps == nr and m % Gk == 0:
        assert flushed_at == nr - 1 - (m % Gk)
