"""Pins of the oracle's mixed-precision parts (MiKV: important tokens at high
precision, the rest at low precision; DiffKV: K8V4 / K4V2 / pruned tiers by
significance).

  - the b-bit codec (b = 2, 4, 8) against an exact-rational restatement of
    its rule (Python Fractions, round-half-even) on numpy's fp32 arithmetic;
    closed-form groups (constant, exact progressions, half-way ties); the
    error bound |x - x_hat| <= scale / 2; b = 2 equals the INT2 codec;
  - the bit-plane word layout against known codes read back by an unpacker
    written here, and the (2, 2) layout equals the INT2 pack bit for bit;
  - attention over the union of segments against torch SDPA (fp64) over an
    independent unpacking; q = 0 gives the mean; segment order is
    irrelevant (the permutation invariance MiKV's regrouping relies on);
  - DiffKV significance: the K = 0 closed form (H_n - H_j) / (n - j) and a
    brute-force softmax matrix per head (max over the group's heads);
  - DiffKV tiers against a brute-force sort, with the counts' rounding;
  - MiKV's printed "avg. 3bit" cache at a half/half split.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

HERE = os.path.dirname(os.path.abspath(__file__))


def _codec_ref(x16, bits):
    top = (1 << bits) - 1
    xf = x16.astype(np.float32)
    mn, mx = xf.min(), xf.max()
    s32 = np.float32(np.float32(mx - mn) / np.float32(top))
    sh = np.float16(s32)
    zh = np.float16(np.float32(mn) + np.float32(0.0))
    codes = []
    for xi in xf:
        if sh == 0:
            codes.append(0)
            continue
        d = np.float32(xi - np.float32(zh))
        q = Fraction(float(d)) / Fraction(float(sh))
        codes.append(min(max(round(q), 0), top))      # round: half to even
    return np.array(codes), int(sh.view(np.uint16)), int(zh.view(np.uint16))


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("G", [16, 32, 128])
def test_codec_bits_vs_rational(oracle, bits, G):
    r = np.random.default_rng(bits * 1000 + G)
    for trial in range(60):
        x = r.standard_normal(G) * np.exp2(r.integers(-12, 10))
        if trial % 3 == 0:
            x[r.integers(G)] *= 40.0                  # an outlier
        x16 = x.astype(np.float16)
        codes, s, z = oracle.quant_group_bits(x16, bits)
        rc, rs, rz = _codec_ref(x16, bits)
        assert (s, z) == (rs, rz)
        assert np.array_equal(codes, rc), (bits, G, trial)


def test_codec_bits_2_equals_int2(oracle):
    r = np.random.default_rng(5)
    for _ in range(200):
        x16 = (r.standard_normal(16) * 3).astype(np.float16)
        a = oracle.quant_group_bits(x16, 2)
        b = oracle.quant_group(x16)
        assert np.array_equal(a[0], b[0]) and a[1:] == b[1:]


@pytest.mark.parametrize("bits", [4, 8])
def test_codec_bits_closed_forms(oracle, bits):
    top = (1 << bits) - 1
    # constant group: scale 0, codes 0, dequant exact
    x = np.full(16, 1.25, np.float16)
    codes, s, z = oracle.quant_group_bits(x, bits)
    assert s == 0 and not codes.any()
    assert oracle.dequant(0, s, z) == np.float32(1.25)
    # exact progression z + c s (s a power of two): codes c, exact dequant
    sv, zv = 2.0 ** -6, -0.75
    cs = np.arange(top + 1) if top < 16 else np.linspace(0, top, 16).round()
    cs = np.concatenate([[0, top], cs]).astype(int)[:16]
    x = (zv + cs * sv).astype(np.float16)
    codes, s, z = oracle.quant_group_bits(x, bits)
    assert np.float16(s and np.uint16(s).view(np.float16)) == np.float16(sv)
    assert np.array_equal(codes, cs)
    for c, xi in zip(codes, x):
        assert oracle.dequant(int(c), s, z) == np.float32(xi)
    # half-way points go to the even code
    halves = np.array([0, top] + [j + 0.5 for j in range(min(top, 14))])
    x = (zv + halves * sv).astype(np.float16)
    codes, s, z = oracle.quant_group_bits(x, bits)
    want = [0, top] + [j + (j & 1) for j in range(min(top, 14))]
    assert np.array_equal(codes, want)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_codec_bits_error_bound(oracle, bits):
    r = np.random.default_rng(bits)
    for _ in range(300):
        x16 = (r.standard_normal(16) * np.exp2(r.integers(-8, 8))).astype(np.float16)
        codes, s, z = oracle.quant_group_bits(x16, bits)
        sh = float(np.uint16(s).view(np.float16))
        for c, xi in zip(codes, x16.astype(np.float32)):
            xh = oracle.dequant(int(c), s, z)
            ulp = float(np.spacing(np.float32(abs(xh)) + np.float32(0)))
            assert abs(float(xi) - float(xh)) <= sh / 2 + ulp / 2


def _unpack_planes_keys(kq, D):
    """kq [P][T][D/16] -> codes [T][D] (plane p = bits 2p..2p+1)."""
    P, T, _ = kq.shape
    codes = np.zeros((T, D), np.int64)
    for p in range(P):
        for c in range(D):
            codes[:, c] |= ((kq[p, :, c // 16].astype(np.int64) >> (2 * (c % 16))) & 3) << (2 * p)
    return codes


def _unpack_planes_values(vq, T):
    """vq [P][T/16][D] -> codes [T][D]."""
    P, _, D = vq.shape
    codes = np.zeros((T, D), np.int64)
    for p in range(P):
        for t in range(T):
            codes[t] |= ((vq[p, t // 16].astype(np.int64) >> (2 * (t % 16))) & 3) << (2 * p)
    return codes


@pytest.mark.parametrize("kb,vb", [(4, 4), (8, 4), (4, 2), (2, 2)])
def test_pack_bits_layout_and_dequant(oracle, kb, vb):
    from bit_quantized_attention_two_amd import synth
    n, D, Gk, Gv = 200, 64, 16, 16
    k, v = synth.gen_kv(kb * 10 + vb, 1, n, D)
    sel = np.sort(np.random.default_rng(kb + vb).choice(n, 70, replace=False)).astype(np.int32)
    out = oracle.pack_unit_bits(k[0], v[0], sel, Gk, Gv, kb, vb)
    mp = 64
    kc = _unpack_planes_keys(out["kq"], D)
    vc = _unpack_planes_values(out["vq"], mp)
    # codes read back equal the codec's codes of each group
    for gi in range(mp // Gk):
        for c in range(D):
            codes, s, z = oracle.quant_group_bits(k[0][sel[gi * Gk:(gi + 1) * Gk], c], kb)
            assert np.array_equal(kc[gi * Gk:(gi + 1) * Gk, c], codes)
            assert (out["ks"][gi, c], out["kz"][gi, c]) == (s, z)
    for p in range(0, mp, 7):
        for G in range(D // Gv):
            codes, s, z = oracle.quant_group_bits(v[0][sel[p], G * Gv:(G + 1) * Gv], vb)
            assert np.array_equal(vc[p, G * Gv:(G + 1) * Gv], codes)
    # the tail stays fp16
    assert np.array_equal(out["kres"], k[0][sel[mp:]].view(np.uint16))
    # dequant_unit = code * scale + zero of the codes read back here
    kh, vh = oracle.dequant_unit(Gk, Gv, kb, vb, mp, out["kq"], out["ks"],
                                 out["kz"], out["vq"], out["vs"], out["vz"])
    ks = out["ks"].view(np.float16).astype(np.float32)
    kz = out["kz"].view(np.float16).astype(np.float32)
    want = (kc.astype(np.float32) * np.repeat(ks, Gk, axis=0) +
            np.repeat(kz, Gk, axis=0)).astype(np.float64)
    assert np.array_equal(kh, want)
    vs = out["vs"].view(np.float16).astype(np.float32)
    vz = out["vz"].view(np.float16).astype(np.float32)
    wantv = (vc.astype(np.float32) * np.repeat(vs, Gv, axis=1) +
             np.repeat(vz, Gv, axis=1)).astype(np.float64)
    assert np.array_equal(vh, wantv)


def test_pack_bits_2_2_equals_int2_pack(oracle):
    from bit_quantized_attention_two_amd import synth
    k, v = synth.gen_kv(3, 1, 300, 128)
    sel = np.sort(np.random.default_rng(1).choice(300, 150, replace=False)).astype(np.int32)
    a = oracle.pack_unit_bits(k[0], v[0], sel, 16, 32, 2, 2)
    b = oracle.pack_unit(k[0], v[0], sel, 16, 32)
    for name in ("ks", "kz", "vs", "vz", "kres", "vres"):
        assert np.array_equal(a[name], b[name]), name
    assert np.array_equal(a["kq"][0], b["kq"]) and np.array_equal(a["vq"][0], b["vq"])


def _mixed(oracle, seed, g=2, D=64, n=300, Gk=16, Gv=16):
    from bit_quantized_attention_two_amd import synth
    B, Hkv = 1, 2
    k, v = synth.gen_kv(seed, B * Hkv, n, D)
    k, v = k.reshape(B, Hkv, n, D), v.reshape(B, Hkv, n, D)
    mc = oracle.OracleMixedCache(B, Hkv, D, Gk, Gv, [(4, 4, 256), (2, 2, 256)])
    r = np.random.default_rng(seed)
    tails_k, tails_v = [], []
    for h in range(Hkv):
        sel = np.sort(r.choice(n, 120, replace=False)).astype(np.int32)
        comp = oracle.complement(sel, n)
        k1, v1 = mc.pack(0, k, v, 0, h, sel)
        k2, v2 = mc.pack(1, k, v, 0, h, comp)
        tails_k.append(np.concatenate([k1, k2]))
        tails_v.append(np.concatenate([v1, v2]))
    mc.set_residual(np.stack(tails_k)[None], np.stack(tails_v)[None])
    q = r.standard_normal((B, Hkv * g, D)).astype(np.float16)
    return mc, q, k, v


def test_mixed_decode_vs_sdpa(oracle):
    mc, q, k, v = _mixed(oracle, 11)
    g, D = 2, 64
    for h in range(2):
        kk, vv = [], []
        for S in mc.segs:
            T = int(S["n"][0, h])
            kc = _unpack_planes_keys(S["kq"][0, h][:, :T], D)
            vc = _unpack_planes_values(S["vq"][0, h][:, :T // 16], T)
            ks = S["ks"][0, h][:T // 16].view(np.float16).astype(np.float64)
            kz = S["kz"][0, h][:T // 16].view(np.float16).astype(np.float64)
            vs = S["vs"][0, h][:T].view(np.float16).astype(np.float64)
            vz = S["vz"][0, h][:T].view(np.float16).astype(np.float64)
            kk.append(kc * np.repeat(ks, 16, axis=0) + np.repeat(kz, 16, axis=0))
            vv.append(vc * np.repeat(vs, 16, axis=1) + np.repeat(vz, 16, axis=1))
        r = mc.n_res
        kk.append(mc.kres[0, h, :r].view(np.float16).astype(np.float64))
        vv.append(mc.vres[0, h, :r].view(np.float16).astype(np.float64))
        K = torch.from_numpy(np.concatenate(kk))
        V = torch.from_numpy(np.concatenate(vv))
        Q = torch.from_numpy(q[0, h * g:(h + 1) * g].astype(np.float64))
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q[None], K[None].expand(1, -1, -1).contiguous(),
            V[None].contiguous())[0].numpy()
        got = mc.decode_unit(q[0, h * g:(h + 1) * g], 0, h)
        np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)
        # q = 0: the mean of every cached value row
        got0 = mc.decode_unit(np.zeros((g, D), np.float16), 0, h)
        np.testing.assert_allclose(got0, np.broadcast_to(V.numpy().mean(0), (g, D)),
                                   rtol=1e-10, atol=1e-12)
    assert mc.segs[0]["n"][0, 0] == 112 and mc.segs[1]["n"][0, 0] == 176
    assert mc.n_res == 8 + 4


def test_mixed_decode_segment_order_irrelevant(oracle):
    mc, q, k, v = _mixed(oracle, 12)
    a = mc.decode_unit(q[0, 0:2], 0, 0)
    mc.segs.reverse()
    b = mc.decode_unit(q[0, 0:2], 0, 0)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


def test_diffkv_score_k0_closed_form(oracle):
    n, D, g = 96, 64, 3
    r = np.random.default_rng(2)
    q = r.standard_normal((g, n, D)).astype(np.float16)
    k = np.zeros((n, D), np.float16)
    v = r.standard_normal((n, D)).astype(np.float16)
    col_h = np.stack([oracle.prefill_rows(q[h:h + 1], k, v, np.arange(n, dtype=np.int32),
                                          want_o=False, want_lse=False)[2]
                      for h in range(g)])
    H = np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, n + 1))])
    want = (H[n] - H[np.arange(n)]) / (n - np.arange(n))
    np.testing.assert_allclose(oracle.diffkv_score(col_h), want, rtol=1e-12)


def test_diffkv_score_bruteforce_max_over_heads(oracle):
    n, D, g = 40, 16, 4
    r = np.random.default_rng(3)
    q = r.standard_normal((g, n, D)).astype(np.float16)
    k = (r.standard_normal((n, D)) * 2).astype(np.float16)
    v = r.standard_normal((n, D)).astype(np.float16)
    col_h = np.stack([oracle.prefill_rows(q[h:h + 1], k, v, np.arange(n, dtype=np.int32),
                                          want_o=False, want_lse=False)[2]
                      for h in range(g)])
    Q = torch.from_numpy(q.astype(np.float64))
    K = torch.from_numpy(k.astype(np.float64))
    S = Q @ K.T / np.sqrt(D)
    S = S.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
    P = torch.softmax(S, dim=-1).numpy()                  # [g][i][j]
    want = (P.sum(axis=1) / (n - np.arange(n))).max(axis=0)
    np.testing.assert_allclose(oracle.diffkv_score(col_h), want, rtol=1e-12)


def _tiers_brute(score, thr_hi, thr_lo, Gk):
    n = score.size
    cap = n // Gk * Gk
    up = lambda c: min((c + Gk - 1) // Gk * Gk, cap)
    c_hi = up(int((score > thr_hi).sum()))
    c_kept = max(up(int((score > thr_lo).sum())), c_hi)
    order = sorted(range(n), key=lambda j: (-score[j], j))
    return sorted(order[:c_hi]), sorted(order[c_hi:c_kept])


@pytest.mark.parametrize("n,Gk", [(1, 16), (16, 16), (100, 16), (257, 32), (512, 16)])
def test_diffkv_tiers_bruteforce(oracle, n, Gk):
    r = np.random.default_rng(n + Gk)
    for kind in range(4):
        if kind == 0:
            s = r.exponential(1.0, n) / n
        elif kind == 1:
            s = r.integers(0, 5, n) / (2.0 * n)          # many ties
        elif kind == 2:
            s = np.full(n, 1.0 / n)
        else:
            s = np.linspace(3.0, 0.01, n) / n
        for a_hi, a_lo in ((1.0, 0.2), (2.0, 0.0), (np.inf, -np.inf), (0.5, 0.5)):
            hi, lo = oracle.diffkv_tiers(s, a_hi / n, a_lo / n, Gk)
            bh, bl = _tiers_brute(s, a_hi / n, a_lo / n, Gk)
            assert list(hi) == bh and list(lo) == bl, (n, kind, a_hi, a_lo)
            assert hi.size % Gk == 0 and lo.size % Gk == 0


def test_diffkv_tiers_special_cases(oracle):
    n, Gk = 64, 16
    s = np.full(n, 1.0 / n)
    hi, lo = oracle.diffkv_tiers(s, np.inf, -np.inf, Gk)   # nothing pruned
    assert hi.size == 0 and list(lo) == list(range(n))
    s = np.linspace(1, 2, n)[::-1].copy()                # decreasing
    hi, lo = oracle.diffkv_tiers(s, 1.5, 1.3, Gk)      # 32 and 45 above
    assert list(hi) == list(range(32)) and list(lo) == list(range(32, 48))


def test_mikv_average_three_bits(oracle):
    """MiKV's rebuttal reports its latency for an average of 3 bits, between
    KIVI's 2-bit and 4-bit (tests/golden/mikv_avg_bits.json): important
    tokens at INT4 and the rest at INT2, half and half, store 3 bits of
    codes per element."""
    g = json.load(open(os.path.join(HERE, "golden", "mikv_avg_bits.json")))
    from bit_quantized_attention_two_amd import synth
    n, D = 512, 128
    k, v = synth.gen_kv(1, 1, n, D)
    sel = np.arange(0, n, 2, dtype=np.int32)
    hi = oracle.pack_unit_bits(k[0], v[0], sel, 16, 16, g["high_bits"], g["high_bits"])
    lo = oracle.pack_unit_bits(k[0], v[0], oracle.complement(sel, n), 16, 16,
                               g["low_bits"], g["low_bits"])
    code_bits = 32 * sum(a[x].size for a in (hi, lo) for x in ("kq", "vq"))
    assert code_bits / (2 * n * D) == g["printed"]["average_bits"]
