"""GPU parity of minikv_decode_attn against the oracle's fp64 decode over
the same (bit-identical) packed cache: |gpu - ref| <= 2e-3 + 1e-3 |ref|."""
import concurrent.futures as cf
import os

import numpy as np
import pytest

import oracle
from bit_quantized_attention_two_amd import synth
from gpu_util import (assert_cache_equal, assert_close, dev16, lib_budgets,
                      require_gpu, say)

pytestmark = pytest.mark.gpu

WORKERS = min(16, os.cpu_count() or 1)


def _build(torch, mk, B, Hkv, g, D, Gk, Gv, n, m, seed, check_bits=True,
           units=None):
    nu = B * Hkv
    k, v = synth.gen_kv(seed, nu, n, D)
    sel = synth.gen_selection(seed, nu, n, m) if m < n else \
        np.tile(np.arange(n, dtype=np.int32), (nu, 1))
    k, v = k.reshape(B, Hkv, n, D), v.reshape(B, Hkv, n, D)
    sel = sel.reshape(B, Hkv, m)
    cap = (m // Gk) * Gk + 256
    dims = mk.make_dims(B, Hkv * g, Hkv, D, Gk, Gv)
    cache = mk.LayerCache(dims, cap)
    mk.pack(dims, dev16(torch, k), dev16(torch, v),
            torch.from_numpy(sel).cuda(), cache)
    oc = oracle.OracleCache(B, Hkv, D, Gk, Gv, cap)
    oc.pack(k, v, sel, units=units, workers=WORKERS)
    if check_bits:
        torch.cuda.synchronize()
        assert_cache_equal(cache, oc, B, Hkv)
    return dims, cache, oc


def _decode_and_compare(torch, mk, dims, cache, oc, q, units=None):
    o = mk.decode_attn(dims, cache, dev16(torch, q)).cpu().numpy()
    B, Hq, D = q.shape
    g = Hq // dims.n_kv_heads
    if units is None:
        units = [(b, h) for b in range(B) for h in range(dims.n_kv_heads)]
    with cf.ThreadPoolExecutor(WORKERS) as ex:
        outs = list(ex.map(lambda u: oc.decode_unit(
            q[u[0], u[1] * g:(u[1] + 1) * g], u[0], u[1]), units))
    for (b, h), ref in zip(units, outs):
        assert_close(o[b, h * g:(h + 1) * g], ref, "decode o[b=%d,kvh=%d]" % (b, h))
    return o


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("g", [1, 2, 4, 8])
@pytest.mark.parametrize("n,m", [(64, 20), (300, 150), (3000, 2100)])
def test_decode_small(D, g, n, m):
    torch, mk = require_gpu()
    B, Hkv = 2, 2
    say("decode", dict(D=D, g=g, n=n, m=m))
    dims, cache, oc = _build(torch, mk, B, Hkv, g, D, 16, 16, n, m, seed=n + g)
    q, _, _ = synth.gen_decode_step(5, 0, 0, B, Hkv * g, Hkv, D)
    _decode_and_compare(torch, mk, dims, cache, oc, q)


@pytest.mark.parametrize("D,g,Gk,Gv", [
    (128, 1, 64, 32), (128, 4, 128, 64), (64, 2, 32, 64), (128, 8, 16, 128),
    (64, 1, 128, 16), (128, 2, 32, 32), (64, 4, 64, 32)])
def test_decode_group_sizes(D, g, Gk, Gv):
    """Key groups of 16..128 tokens and value groups of 16..128 channels:
    value groups wider than 16 channels repeat their scale per 16-channel
    part; key groups wider than 16 tokens span several key tiles."""
    torch, mk = require_gpu()
    B, Hkv, n, m = 2, 2, 3000, 2100
    say("decode-groups", dict(D=D, g=g, Gk=Gk, Gv=Gv))
    dims, cache, oc = _build(torch, mk, B, Hkv, g, D, Gk, Gv, n, m,
                             seed=7 * Gk + Gv + g)
    for s_ in range(3):
        q, kn, vn = synth.gen_decode_step(11, 0, s_, B, Hkv * g, Hkv, D)
        mk.append(dims, cache, dev16(torch, kn), dev16(torch, vn))
        oc.append(kn, vn)
        _decode_and_compare(torch, mk, dims, cache, oc, q)


def test_decode_group32_keys_and_residual_only():
    torch, mk = require_gpu()
    # tiny single-layer workload: D 64, 4 heads, key groups of 32 tokens
    dims, cache, oc = _build(torch, mk, 1, 4, 1, 64, 32, 16, 256, 128, seed=1)
    q, _, _ = synth.gen_decode_step(1, 0, 0, 1, 4, 4, 64)
    _decode_and_compare(torch, mk, dims, cache, oc, q)
    # fewer selected tokens than one key group: residual only
    dims, cache, oc = _build(torch, mk, 1, 2, 4, 128, 16, 16, 40, 11, seed=2)
    assert cache.n_packed == 0 and cache.n_res == 11
    q, _, _ = synth.gen_decode_step(2, 0, 0, 1, 8, 2, 128)
    _decode_and_compare(torch, mk, dims, cache, oc, q)


def test_decode_after_appends_and_determinism():
    torch, mk = require_gpu()
    B, Hkv, g, D = 1, 4, 2, 128
    dims, cache, oc = _build(torch, mk, B, Hkv, g, D, 16, 16, 900, 500, seed=3)
    for s in range(140):                        # crosses one flush
        q, kn, vn = synth.gen_decode_step(3, 0, s, B, Hkv * g, Hkv, D)
        mk.append(dims, cache, dev16(torch, kn), dev16(torch, vn))
        oc.append(kn, vn)
        if s in (0, 10, 139) or oc.n_res == 0:
            o1 = _decode_and_compare(torch, mk, dims, cache, oc, q)
            o2 = mk.decode_attn(dims, cache, dev16(torch, q)).cpu().numpy()
            assert np.array_equal(o1.view(np.uint16), o2.view(np.uint16))


@pytest.mark.parametrize("Hkv", [4, 3])
def test_decode_shared_workspace(Hkv):
    """Two caches of different capacities and a residual-only one, with the
    same dims, share one workspace across interleaved calls (plain and
    fused-append forms): every call must match the oracle."""
    torch, mk = require_gpu()
    B, g, D = 2, 2, 128
    say("decode-shared-ws", dict(B=B, Hkv=Hkv, g=g))
    a = _build(torch, mk, B, Hkv, g, D, 16, 16, 1500, 900, seed=21)
    b = _build(torch, mk, B, Hkv, g, D, 16, 16, 3000, 2100, seed=22)
    c = _build(torch, mk, B, Hkv, g, D, 16, 16, 40, 9, seed=23)   # residual only
    dims = a[0]
    ws = torch.zeros(max(mk.decode_ws_bytes(dims, x[1].capacity) for x in (a, b, c)),
                     dtype=torch.uint8, device="cuda")
    for s in range(6):
        for (_, cache, oc) in ((a if s % 2 else b), c, (b if s % 2 else a)):
            q, kn, vn = synth.gen_decode_step(24, 0, s, B, Hkv * g, Hkv, D)
            if s >= 3:
                o = mk.append_decode(dims, cache, dev16(torch, kn), dev16(torch, vn),
                                     dev16(torch, q), ws=ws).cpu().numpy()
                oc.append(kn, vn)
            else:
                o = mk.decode_attn(dims, cache, dev16(torch, q), ws=ws).cpu().numpy()
            units = [(bb, h) for bb in range(B) for h in range(Hkv)]
            for (bb, h) in units:
                ref = oc.decode_unit(q[bb, h * g:(h + 1) * g], bb, h)
                assert_close(o[bb, h * g:(h + 1) * g], ref, "s%d b%d h%d" % (s, bb, h))


def test_decode_empty_cache_is_an_error():
    torch, mk = require_gpu()
    dims = mk.make_dims(1, 2, 2, 128)
    cache = mk.LayerCache(dims, 64)
    q = torch.zeros((1, 2, 128), dtype=torch.float16, device="cuda")
    with pytest.raises(mk.MiniKVError) as e:
        mk.decode_attn(dims, cache, q)
    assert e.value.status == mk.EINVAL


@pytest.mark.parametrize("cfg_id", [3, 4, 5])
def test_decode_full_size(cfg_id):
    """Decode at the workloads' real sizes: the packed cache of one layer
    (n/4 heavy hitters + n/4 recent tokens per unit, layer 0 budget), every
    unit (configs 4, 5) or 48 sampled units (config 3) against the oracle."""
    torch, mk = require_gpu()
    from bit_quantized_attention_two_amd import configs
    c = configs.get(cfg_id)
    B, Hkv, g, D, n = c["B"], c["Hkv"], c["g"], c["D"], c["n"]
    ks, r = lib_budgets(mk, c)
    m = int(ks[0]) + r
    say("decode-full", dict(cfg=cfg_id, B=B, Hkv=Hkv, g=g, n=n, m=m))
    units = [(b, h) for b in range(B) for h in range(Hkv)]
    if len(units) > 48:
        rr = np.random.default_rng(cfg_id)
        units = [units[i] for i in sorted(rr.choice(len(units), 48, replace=False))]
    dims, cache, oc = _build(torch, mk, B, Hkv, g, D, 16, 16, n, m,
                             seed=100 + cfg_id, check_bits=False, units=units)
    q, kn, vn = synth.gen_decode_step(cfg_id, 0, 0, B, Hkv * g, Hkv, D)
    mk.append(dims, cache, dev16(torch, kn), dev16(torch, vn))
    oc.append(kn, vn)
    torch.cuda.synchronize()
    # bit-exact packed region on the sampled units
    from gpu_util import cache_to_numpy
    gc = cache_to_numpy(cache)
    for b, h in units:
        u = b * Hkv + h
        for gname, oname in (("kq", "kq"), ("k_scale", "ks"), ("k_zero", "kz"),
                             ("vq", "vq"), ("v_scale", "vs"), ("v_zero", "vz"),
                             ("k_res", "kres"), ("v_res", "vres")):
            assert np.array_equal(gc[gname][u], getattr(oc, oname)[b, h]), \
                (gname, b, h)
    _decode_and_compare(torch, mk, dims, cache, oc, q, units)


@pytest.mark.parametrize("D,g,Gv", [(128, 1, 16), (128, 2, 16), (64, 2, 32),
                                    (128, 1, 64)])
def test_decode_multi_batch_waves(D, g, Gv):
    """Enough units (8 x 32 kv heads) that the split size grows past the
    minimum: each wave then walks several 64-token key batches and many
    value steps, the form the small tests (4 units, single-batch waves)
    never reach for g <= 2.  16 sampled units against the oracle."""
    torch, mk = require_gpu()
    B, Hkv, n, m = 8, 32, 2200, 2100
    say("decode-multibatch", dict(D=D, g=g, Gv=Gv))
    units = [(b, h) for b in range(B) for h in range(Hkv)]
    rr = np.random.default_rng(D + g + Gv)
    units = [units[i] for i in sorted(rr.choice(len(units), 16, replace=False))]
    dims, cache, oc = _build(torch, mk, B, Hkv, g, D, 16, Gv, n, m,
                             seed=40 + g + Gv, check_bits=False, units=units)
    q, kn, vn = synth.gen_decode_step(7, 0, 0, B, Hkv * g, Hkv, D)
    mk.append(dims, cache, dev16(torch, kn), dev16(torch, vn))
    oc.append(kn, vn)
    _decode_and_compare(torch, mk, dims, cache, oc, q, units)


@pytest.mark.parametrize("g,D", [(1, 128), (4, 128), (8, 128), (1, 64), (8, 64)])
def test_decode_full_and_partial_wave_shares(g, D):
    """Wave shares of 256 tokens (eight full ones per unit) and one of 240
    (its last 32-token value step half past the end): the shares that run
    as straight-line code, full and partial, next to a short one; 256 units
    so that the split plan picks 256-token shares (the 12-wave form at
    g = 4, the 4-wave form at g = 1 and 8; at D = 64 too).  16 sampled
    units against the oracle."""
    torch, mk = require_gpu()
    B, Hkv, n = 8, 32, 2400
    m = 8 * 256 + 240 + 5                         # 2288 packed + 5 residual
    say("decode-full-partial-shares", dict(g=g, D=D, n=n, m=m))
    units = [(b, h) for b in range(B) for h in range(Hkv)]
    rr = np.random.default_rng(70 + g + D)
    units = [units[i] for i in sorted(rr.choice(len(units), 16, replace=False))]
    dims, cache, oc = _build(torch, mk, B, Hkv, g, D, 16, 16, n, m,
                             seed=60 + g + D, check_bits=False, units=units)
    q, kn, vn = synth.gen_decode_step(8, 0, 0, B, Hkv * g, Hkv, D)
    mk.append(dims, cache, dev16(torch, kn), dev16(torch, vn))
    oc.append(kn, vn)
    _decode_and_compare(torch, mk, dims, cache, oc, q, units)


@pytest.mark.parametrize("n,m,D,Gk,Gv", [
    (41000, 40000, 128, 16, 16), (24000, 23400, 128, 16, 16),
    (81000, 80000, 128, 16, 16), (71000, 70000, 128, 16, 16),
    (41000, 40000, 64, 16, 16), (41000, 40000, 128, 64, 32)])
def test_decode_one_round_gqa(n, m, D, Gk, Gv):
    """g = 4 calls in the one-round 12-wave form, 8 kv heads: 27 splits of
    128-token wave shares (the 4-wave form would need 512-token splits), 31
    of 64, and, where the 4-wave grid would give some CUs a third block,
    30 splits of 224 (seven 32-token value steps, an odd count) and 31 of
    192; at D = 128 and 64, and with key groups of 64 tokens and value
    groups of 32 channels; every unit against the oracle."""
    torch, mk = require_gpu()
    B, Hkv, g = 1, 8, 4
    say("decode-one-round-gqa", dict(n=n, m=m, D=D, Gk=Gk, Gv=Gv))
    dims, cache, oc = _build(torch, mk, B, Hkv, g, D, Gk, Gv, n, m,
                             seed=90 + m % 7, check_bits=False)
    q, kn, vn = synth.gen_decode_step(9, 0, 0, B, Hkv * g, Hkv, D)
    mk.append(dims, cache, dev16(torch, kn), dev16(torch, vn))
    oc.append(kn, vn)
    _decode_and_compare(torch, mk, dims, cache, oc, q)


@pytest.mark.parametrize("g,D,B,Hkv,n,m", [
    (1, 128, 2, 2, 700, 333), (4, 128, 2, 2, 700, 333), (2, 64, 2, 2, 700, 333),
    # 32 kv heads x 8 splits of 3072 tokens: the one-round 12-wave GQA form,
    # with the residual on the last split's idle waves
    (4, 128, 4, 8, 24000, 23400)])
def test_append_decode_equals_separate_calls(g, D, B, Hkv, n, m):
    """The fused entry point gives the same bits as minikv_append followed by
    minikv_decode_attn, across a residual flush, and leaves the same cache."""
    torch, mk = require_gpu()
    from gpu_util import cache_to_numpy
    dims, ca, _ = _build(torch, mk, B, Hkv, g, D, 16, 16, n, m, seed=21,
                         check_bits=False, units=[(0, 0)])
    _, cb, _ = _build(torch, mk, B, Hkv, g, D, 16, 16, n, m, seed=21,
                      check_bits=False, units=[(0, 0)])
    say("append_decode", dict(g=g, D=D, B=B, Hkv=Hkv, m=m))
    for s in range(140):
        q, kn, vn = synth.gen_decode_step(21, 0, s, B, Hkv * g, Hkv, D)
        q, kn, vn = dev16(torch, q), dev16(torch, kn), dev16(torch, vn)
        mk.append(dims, ca, kn, vn)
        oa = mk.decode_attn(dims, ca, q)
        ob = mk.append_decode(dims, cb, kn, vn, q)
        assert (ca.n_packed, ca.n_res) == (cb.n_packed, cb.n_res)
        if s % 23 == 0 or ca.n_res in (0, 1):
            torch.cuda.synchronize()
            assert torch.equal(oa, ob), s
            xa, xb = cache_to_numpy(ca), cache_to_numpy(cb)
            for name in xa:
                assert np.array_equal(xa[name], xb[name]), (s, name)


@pytest.mark.parametrize("B,Hkv,g,D,Gk,Gv,n,m", [
    (1, 2, 1, 128, 16, 16, 900, 500),     # single-batch waves
    (1, 2, 4, 64, 32, 16, 900, 500),
    (2, 2, 2, 128, 16, 32, 700, 330),
    (8, 32, 1, 128, 16, 16, 2200, 2100),  # multi-batch waves
    (9, 32, 4, 128, 16, 16, 2400, 2293),  # 256- and 240-token shares, 4-wave
])                                        # blocks for both calls (288 units)
def test_decode_mass_matches_oracle(B, Hkv, g, D, Gk, Gv, n, m):
    """Persistence audit: minikv_decode_attn_mass gives decode_attn's o bit
    for bit, and accumulates every cached token's attention weight (summed
    over the kv head's query heads) in cache order; over steps that cross a
    residual flush the accumulated mass matches the oracle's weights summed
    the same way, within 1e-3 relative + 1e-6 per step, and sums to g per
    step."""
    torch, mk = require_gpu()
    say("decode-mass", dict(B=B, Hkv=Hkv, g=g, D=D, Gk=Gk, Gv=Gv, n=n, m=m))
    units = [(b, h) for b in range(B) for h in range(Hkv)]
    if len(units) > 8:
        rr = np.random.default_rng(m)
        units = [units[i] for i in sorted(rr.choice(len(units), 8, replace=False))]
    dims, cache, oc = _build(torch, mk, B, Hkv, g, D, Gk, Gv, n, m,
                             seed=60 + g + D, check_bits=False, units=units)
    stride = cache.capacity + dims.residual_cap
    mass = torch.zeros(B, Hkv, stride, dtype=torch.float32, device="cuda")
    ref = np.zeros((B, Hkv, stride))
    steps = 0
    for s_ in range(132 - cache.n_res):          # the last step flushes
        q, kn, vn = synth.gen_decode_step(13, 0, s_, B, Hkv * g, Hkv, D)
        mk.append(dims, cache, dev16(torch, kn), dev16(torch, vn))
        oc.append(kn, vn)
        if s_ % 40 and oc.n_res != 0:
            continue
        qd = dev16(torch, q)
        o = mk.decode_attn_mass(dims, cache, qd, mass)
        o_plain = mk.decode_attn(dims, cache, qd)
        assert torch.equal(o.view(torch.int16), o_plain.view(torch.int16))
        steps += 1
        T = oc.n_packed + oc.n_res
        with cf.ThreadPoolExecutor(WORKERS) as ex:
            outs = list(ex.map(lambda u: oc.decode_unit(
                q[u[0], u[1] * g:(u[1] + 1) * g], u[0], u[1], with_mass=True),
                units))
        for (b, h), (ro, rm) in zip(units, outs):
            assert_close(o.cpu().numpy()[b, h * g:(h + 1) * g], ro,
                         "decode o[b=%d,kvh=%d]" % (b, h))
            ref[b, h, :T] += rm
    got = mass.cpu().numpy().astype(np.float64)
    for b, h in units:
        err = np.abs(got[b, h] - ref[b, h])
        bad = err > 1e-3 * np.abs(ref[b, h]) + 1e-6 * steps
        assert not bad.any(), ("mass", b, h, int(np.argmax(err)), err.max())
        assert abs(got[b, h].sum() - g * steps) <= 1e-4 * g * steps
    say("decode-mass steps", steps)
