"""numpy wrappers around the oracle's C functions (ctypes; the GIL is released
during each call, so callers may run units on a thread pool).

Arrays of fp16 are passed as their raw uint16 bit patterns.  Shapes follow the
cache layout the oracle defines (see ``OracleCache``).
"""
import ctypes
import os

import numpy as np

from .build_oracle import build, lib_path

_lib = None


def _load():
    global _lib
    if _lib is None:
        path = lib_path()
        if not os.path.exists(path):
            build()
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32 = ctypes.c_int
        lib.oracle_h2d.argtypes = [ctypes.c_uint16]
        lib.oracle_h2d.restype = ctypes.c_double
        lib.oracle_f2h_rne.argtypes = [ctypes.c_float]
        lib.oracle_f2h_rne.restype = ctypes.c_uint16
        lib.oracle_quant_group.argtypes = [P, i32, ctypes.c_long, P, P, P]
        lib.oracle_quant_group.restype = None
        lib.oracle_dequant.argtypes = [i32, ctypes.c_uint16, ctypes.c_uint16]
        lib.oracle_dequant.restype = ctypes.c_float
        lib.oracle_budgets.argtypes = [i32] * 8 + [P, P]
        lib.oracle_budgets.restype = i32
        lib.oracle_prefill_rows.argtypes = [i32, i32, i32, P, P, P, P, i32,
                                            P, P, P]
        lib.oracle_prefill_rows.restype = None
        lib.oracle_select.argtypes = [i32, P, i32, i32, P]
        lib.oracle_select.restype = i32
        lib.oracle_pack_unit.argtypes = [i32, i32, i32, P, P, P, i32] + [P] * 8
        lib.oracle_pack_unit.restype = i32
        lib.oracle_decode_unit.argtypes = [i32, i32, i32, i32, P, i32] + \
            [P] * 6 + [i32, P, P, P, P]
        lib.oracle_decode_unit.restype = i32
        lib.oracle_cache_bytes.argtypes = [i32, i32, i32, i32, i32,
                                           ctypes.c_double, i32, i32, P]
        lib.oracle_cache_bytes.restype = ctypes.c_double
        lib.oracle_quant_group_bits.argtypes = [P, i32, ctypes.c_long, i32,
                                                P, P, P]
        lib.oracle_quant_group_bits.restype = None
        lib.oracle_pack_unit_bits.argtypes = [i32] * 5 + [P, P, P, i32] + [P] * 8
        lib.oracle_pack_unit_bits.restype = i32
        lib.oracle_dequant_unit.argtypes = [i32] * 7 + [P] * 8
        lib.oracle_dequant_unit.restype = i32
        lib.oracle_attend.argtypes = [i32, i32, P, i32, P, P, P]
        lib.oracle_attend.restype = i32
        lib.oracle_diffkv_score.argtypes = [i32, i32, P, P]
        lib.oracle_diffkv_score.restype = None
        lib.oracle_diffkv_tiers.argtypes = [i32, P, ctypes.c_double,
                                            ctypes.c_double, i32, P, P, P]
        lib.oracle_diffkv_tiers.restype = i32
        _lib = lib
    return _lib


def _ptr(a):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def _u16(a):
    a = np.asarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    assert a.dtype == np.uint16
    return np.ascontiguousarray(a)


# ----------------------------------------------------------------- scalars --

def h2d(h):
    return _load().oracle_h2d(int(h))


def f2h_rne(x):
    return _load().oracle_f2h_rne(float(np.float32(x)))


def dequant(code, scale_bits, zero_bits):
    return np.float32(_load().oracle_dequant(int(code), int(scale_bits),
                                             int(zero_bits)))


def quant_group(x):
    """One INT2 group: returns (codes uint8[G], scale bits, zero bits)."""
    x = _u16(x).ravel()
    codes = np.zeros(x.size, np.uint8)
    s = np.zeros(1, np.uint16)
    z = np.zeros(1, np.uint16)
    _load().oracle_quant_group(_ptr(x), x.size, 1, _ptr(codes), _ptr(s),
                               _ptr(z))
    return codes, int(s[0]), int(z[0])


# ----------------------------------------------------------------- budgets --

def budgets(n, n_layers, depth=7, pyramid=True, hh=(1, 4), rw=(1, 4)):
    """Per-layer heavy-hitter budgets k_l and the recent window r."""
    k = np.zeros(n_layers, np.int32)
    r = np.zeros(1, np.int32)
    rc = _load().oracle_budgets(n, n_layers, hh[0], hh[1], rw[0], rw[1],
                                depth, 1 if pyramid else 0, _ptr(k), _ptr(r))
    if rc != 0:
        raise ValueError("bad budget arguments")
    return k, int(r[0])


# ----------------------------------------------------------------- prefill --

def prefill_rows(q, k, v, rows, want_o=True, want_lse=True, want_col=True):
    """One unit: q [g][n][D], k/v [n][D] (fp16 or uint16).  Evaluates the
    listed query rows; returns (o [g][len(rows)][D], lse [g][len(rows)],
    col [n] = contributions of those rows), fp64; unwanted parts are None."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    g, n, D = q.shape
    assert k.shape == (n, D) and v.shape == (n, D)
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    nr = rows.size
    o = np.zeros((g, nr, D), np.float64) if want_o else None
    lse = np.zeros((g, nr), np.float64) if want_lse else None
    col = np.zeros(n, np.float64) if want_col else None
    _load().oracle_prefill_rows(
        n, D, g, _ptr(q), _ptr(k), _ptr(v), _ptr(rows), nr,
        _ptr(o) if o is not None else None,
        _ptr(lse) if lse is not None else None,
        _ptr(col) if col is not None else None)
    return o, lse, col


def prefill_unit(q, k, v):
    n = np.asarray(q).shape[1]
    return prefill_rows(q, k, v, np.arange(n, dtype=np.int32))


# ------------------------------------------------------------------ select --

def select(col, n_hh, n_recent):
    col = np.ascontiguousarray(col, dtype=np.float64)
    n = col.size
    sel = np.zeros(max(n_hh + n_recent, 1), np.int32)
    rc = _load().oracle_select(n, _ptr(col), n_hh, n_recent, _ptr(sel))
    if rc != 0:
        raise ValueError("bad selection arguments")
    return sel[:n_hh + n_recent]


# -------------------------------------------------------------------- pack --

def pack_unit(k, v, sel, Gk, Gv):
    """Pack one unit.  Returns dict of kq, ks, kz, vq, vs, vz, kres, vres."""
    k, v = _u16(k), _u16(v)
    n, D = k.shape
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    m = sel.size
    mp = (m // Gk) * Gk
    out = dict(
        kq=np.zeros((mp, D // 16), np.uint32),
        ks=np.zeros((mp // Gk, D), np.uint16),
        kz=np.zeros((mp // Gk, D), np.uint16),
        vq=np.zeros((mp // 16, D), np.uint32),
        vs=np.zeros((mp, D // Gv), np.uint16),
        vz=np.zeros((mp, D // Gv), np.uint16),
        kres=np.zeros((m - mp, D), np.uint16),
        vres=np.zeros((m - mp, D), np.uint16),
    )
    rc = _load().oracle_pack_unit(
        D, Gk, Gv, _ptr(k), _ptr(v), _ptr(sel), m,
        *[_ptr(out[x]) for x in ("kq", "ks", "kz", "vq", "vs", "vz",
                                  "kres", "vres")])
    if rc != mp:
        raise ValueError("bad pack arguments")
    return out


# ------------------------------------------------------------------ decode --

def decode_unit(q, Gk, Gv, n_packed, kq, ks, kz, vq, vs, vz, n_res, kres,
                vres, with_mass=False):
    """q [g][D]; packed arrays of one unit (first n_packed tokens used);
    kres/vres [>=n_res][D].  Returns o [g][D] fp64, and with_mass also the
    attention weight of every cached token summed over the g heads,
    [n_packed + n_res] fp64 in cache order."""
    q = _u16(q)
    g, D = q.shape
    arrs = [np.ascontiguousarray(a) for a in (kq, ks, kz, vq, vs, vz)]
    kres, vres = _u16(kres), _u16(vres)
    o = np.zeros((g, D), np.float64)
    mass = np.zeros(max(n_packed + n_res, 1), np.float64) if with_mass else None
    rc = _load().oracle_decode_unit(D, g, Gk, Gv, _ptr(q), n_packed,
                                    *[_ptr(a) for a in arrs], n_res,
                                    _ptr(kres), _ptr(vres), _ptr(o),
                                    _ptr(mass) if with_mass else None)
    if rc != 0:
        raise ValueError("bad decode arguments")
    return (o, mass[:n_packed + n_res]) if with_mass else o


# -------------------------------------------------------------- cache size --

def cache_bytes(n_layers, n_heads, head_dim, lprompt, lgen, budget_frac,
                bits=2, group=16):
    full = np.zeros(1, np.float64)
    b = _load().oracle_cache_bytes(n_layers, n_heads, head_dim, lprompt, lgen,
                                   budget_frac, bits, group, _ptr(full))
    return b, float(full[0])


# ------------------------------------------------------- layer-level cache --

class OracleCache:
    """One layer's compressed cache for B x Hkv units, in the layout the
    oracle defines:

      kq [B][Hkv][cap][D/16] uint32   word (t, j): channels 16j..16j+15 of
                                       token t, channel 16j+e at bits 2e..2e+1
      ks, kz [B][Hkv][cap/Gk][D]      fp16 bits, one per key group/channel
      vq [B][Hkv][cap/16][D] uint32   word (w, c): tokens 16w..16w+15 of
                                       channel c, token 16w+e at bits 2e..
      vs, vz [B][Hkv][cap][D/Gv]      fp16 bits, one per token/channel group
      kres, vres [B][Hkv][nr][D]      fp16 residual (KIVI streaming buffer)
    """

    def __init__(self, B, Hkv, D, Gk, Gv, capacity, residual_cap=128):
        assert capacity % Gk == 0 and residual_cap % Gk == 0
        self.B, self.Hkv, self.D, self.Gk, self.Gv = B, Hkv, D, Gk, Gv
        self.cap, self.nr = capacity, residual_cap
        self.kq = np.zeros((B, Hkv, capacity, D // 16), np.uint32)
        self.ks = np.zeros((B, Hkv, capacity // Gk, D), np.uint16)
        self.kz = np.zeros_like(self.ks)
        self.vq = np.zeros((B, Hkv, capacity // 16, D), np.uint32)
        self.vs = np.zeros((B, Hkv, capacity, D // Gv), np.uint16)
        self.vz = np.zeros_like(self.vs)
        self.kres = np.zeros((B, Hkv, residual_cap, D), np.uint16)
        self.vres = np.zeros_like(self.kres)
        self.n_packed = 0
        self.n_res = 0

    def _store(self, b, h, at, out):
        Gk, D = self.Gk, self.D
        mp = out["kq"].shape[0]
        self.kq[b, h, at:at + mp] = out["kq"]
        self.ks[b, h, at // Gk:(at + mp) // Gk] = out["ks"]
        self.kz[b, h, at // Gk:(at + mp) // Gk] = out["kz"]
        self.vq[b, h, at // 16:(at + mp) // 16] = out["vq"]
        self.vs[b, h, at:at + mp] = out["vs"]
        self.vz[b, h, at:at + mp] = out["vz"]
        return mp

    def pack(self, k, v, sel, units=None, workers=1):
        """k, v [B][Hkv][n][D]; sel [B][Hkv][m] ascending.  `units` limits
        the work to the listed (b, h) pairs (the others stay zero);
        `workers` > 1 runs units on a thread pool (same arithmetic)."""
        k, v = _u16(k), _u16(v)
        sel = np.asarray(sel, np.int32)
        m = sel.shape[-1]
        mp = (m // self.Gk) * self.Gk
        if mp > self.cap or m - mp > self.nr:
            raise ValueError("capacity exceeded")
        if units is None:
            units = [(b, h) for b in range(self.B) for h in range(self.Hkv)]

        def one(bh):
            b, h = bh
            out = pack_unit(k[b, h], v[b, h], sel[b, h], self.Gk, self.Gv)
            self._store(b, h, 0, out)
            self.kres[b, h, :m - mp] = out["kres"]
            self.vres[b, h, :m - mp] = out["vres"]

        if workers > 1:
            import concurrent.futures as cf
            with cf.ThreadPoolExecutor(workers) as ex:
                list(ex.map(one, units))
        else:
            for bh in units:
                one(bh)
        self.n_packed, self.n_res = mp, m - mp

    def append(self, k_new, v_new):
        """k_new, v_new [B][Hkv][D]; flushes the residual into the packed
        region when it reaches residual_cap tokens (KIVI's nr = 128)."""
        k_new, v_new = _u16(k_new), _u16(v_new)
        if self.n_res + 1 == self.nr and self.n_packed + self.nr > self.cap:
            raise ValueError("capacity exceeded")
        self.kres[:, :, self.n_res] = k_new
        self.vres[:, :, self.n_res] = v_new
        self.n_res += 1
        if self.n_res == self.nr:
            ident = np.arange(self.nr, dtype=np.int32)
            for b in range(self.B):
                for h in range(self.Hkv):
                    out = pack_unit(self.kres[b, h], self.vres[b, h], ident,
                                    self.Gk, self.Gv)
                    self._store(b, h, self.n_packed, out)
            self.n_packed += self.nr
            self.n_res = 0

    def decode(self, q, units=None):
        """q [B][Hq][D] -> o [B][Hq][D] fp64 (rows of unlisted units = nan)."""
        q = _u16(q)
        B, Hq, D = q.shape
        g = Hq // self.Hkv
        o = np.full((B, Hq, D), np.nan)
        if units is None:
            units = [(b, h) for b in range(B) for h in range(self.Hkv)]
        for b, h in units:
            o[b, h * g:(h + 1) * g] = self.decode_unit(q[b, h * g:(h + 1) * g],
                                                       b, h)
        return o

    def decode_unit(self, qg, b, h, with_mass=False):
        return decode_unit(qg, self.Gk, self.Gv, self.n_packed,
                           self.kq[b, h], self.ks[b, h], self.kz[b, h],
                           self.vq[b, h], self.vs[b, h], self.vz[b, h],
                           self.n_res, self.kres[b, h], self.vres[b, h],
                           with_mass)


# --------------------------------------------------- mixed-precision caches --
# MiKV ("Don't Discard, but Keep It Small": important tokens at high
# precision, the others kept at low precision, regrouped by precision) and
# DiffKV (K8V4 / K4V2 / pruned tiers by significance, decided per head).

def quant_group_bits(x, bits):
    """One b-bit group: (codes uint8[G], scale bits, zero bits)."""
    x = _u16(x).ravel()
    codes = np.zeros(x.size, np.uint8)
    s = np.zeros(1, np.uint16)
    z = np.zeros(1, np.uint16)
    _load().oracle_quant_group_bits(_ptr(x), x.size, 1, int(bits), _ptr(codes),
                                    _ptr(s), _ptr(z))
    return codes, int(s[0]), int(z[0])


def pack_unit_bits(k, v, sel, Gk, Gv, key_bits, value_bits):
    """Pack one unit at key_bits / value_bits (bit planes of the INT2 word
    layout).  Returns dict kq [Pk][mp][D/16], ks, kz [mp/Gk][D],
    vq [Pv][mp/16][D], vs, vz [mp][D/Gv], kres, vres [m - mp][D]."""
    k, v = _u16(k), _u16(v)
    n, D = k.shape
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    m = sel.size
    mp = (m // Gk) * Gk
    out = dict(
        kq=np.zeros((key_bits // 2, mp, D // 16), np.uint32),
        ks=np.zeros((mp // Gk, D), np.uint16),
        kz=np.zeros((mp // Gk, D), np.uint16),
        vq=np.zeros((value_bits // 2, mp // 16, D), np.uint32),
        vs=np.zeros((mp, D // Gv), np.uint16),
        vz=np.zeros((mp, D // Gv), np.uint16),
        kres=np.zeros((m - mp, D), np.uint16),
        vres=np.zeros((m - mp, D), np.uint16),
    )
    rc = _load().oracle_pack_unit_bits(
        D, Gk, Gv, key_bits, value_bits, _ptr(k), _ptr(v), _ptr(sel), m,
        *[_ptr(out[x]) for x in ("kq", "ks", "kz", "vq", "vs", "vz",
                                  "kres", "vres")])
    if rc != mp:
        raise ValueError("bad pack arguments")
    return out


def dequant_unit(Gk, Gv, key_bits, value_bits, n_packed, kq, ks, kz, vq, vs,
                 vz):
    """Dequantised K, V [n_packed][D] (fp32 values in fp64) of one unit's
    segment; kq [Pk][cap][D/16], vq [Pv][cap/16][D], metadata for cap."""
    kq, vq = np.ascontiguousarray(kq), np.ascontiguousarray(vq)
    ks, kz, vs, vz = (np.ascontiguousarray(a) for a in (ks, kz, vs, vz))
    cap, D = kq.shape[1], kq.shape[2] * 16
    kh = np.zeros((max(n_packed, 1), D), np.float64)
    vh = np.zeros_like(kh)
    rc = _load().oracle_dequant_unit(D, Gk, Gv, key_bits, value_bits, n_packed,
                                     cap, _ptr(kq), _ptr(ks), _ptr(kz),
                                     _ptr(vq), _ptr(vs), _ptr(vz), _ptr(kh),
                                     _ptr(vh))
    if rc != 0:
        raise ValueError("bad dequant arguments")
    return kh[:n_packed], vh[:n_packed]


def attend(q, kh, vh):
    """Softmax attention of q [g][D] (fp16) over rows kh, vh [T][D] (fp64)."""
    q = _u16(q)
    g, D = q.shape
    kh = np.ascontiguousarray(kh, np.float64)
    vh = np.ascontiguousarray(vh, np.float64)
    o = np.zeros((g, D), np.float64)
    rc = _load().oracle_attend(D, g, _ptr(q), kh.shape[0], _ptr(kh), _ptr(vh),
                               _ptr(o))
    if rc != 0:
        raise ValueError("bad attend arguments")
    return o


def complement(sel, n):
    """The tokens of [0, n) not in sel, ascending: MiKV's low-precision
    group (the tokens an eviction method would drop)."""
    keep = np.ones(n, bool)
    keep[np.asarray(sel, np.int64)] = False
    return np.nonzero(keep)[0].astype(np.int32)


def diffkv_score(col_h):
    """col_h [g][n] per-head column sums -> significance [n] (average
    received attention, max over the group's heads)."""
    col_h = np.ascontiguousarray(col_h, np.float64)
    g, n = col_h.shape
    score = np.zeros(n, np.float64)
    _load().oracle_diffkv_score(n, g, _ptr(col_h), _ptr(score))
    return score


def diffkv_tiers(score, thr_hi, thr_lo, Gk):
    """(high tier, low tier) index arrays, ascending, from significance
    scores and the two thresholds."""
    score = np.ascontiguousarray(score, np.float64)
    n = score.size
    hi = np.zeros(max(n, 1), np.int32)
    lo = np.zeros(max(n, 1), np.int32)
    cnt = np.zeros(2, np.int32)
    rc = _load().oracle_diffkv_tiers(n, _ptr(score), float(thr_hi),
                                     float(thr_lo), Gk, _ptr(hi), _ptr(lo),
                                     _ptr(cnt))
    if rc != 0:
        raise ValueError("bad tier arguments")
    return hi[:cnt[0]], lo[:cnt[1]]


class OracleMixedCache:
    """One layer's mixed-precision cache for B x Hkv units: packed segments
    of given key/value bits (each unit may hold its own count of packed
    tokens in a segment) plus one fp16 residual.  Segment arrays:

      kq [B][Hkv][Pk][cap][D/16], ks, kz [B][Hkv][cap/Gk][D]
      vq [B][Hkv][Pv][cap/16][D], vs, vz [B][Hkv][cap][D/Gv]
      n  [B][Hkv]   packed tokens per unit (multiples of Gk)

    A residual flush quantises the residual into segment `flush_seg`."""

    def __init__(self, B, Hkv, D, Gk, Gv, segs, residual_cap=128, flush_seg=0):
        self.B, self.Hkv, self.D, self.Gk, self.Gv = B, Hkv, D, Gk, Gv
        self.nr, self.flush_seg = residual_cap, flush_seg
        self.segs = []
        for kb, vb, cap in segs:
            assert cap % Gk == 0 and cap % 16 == 0
            self.segs.append(dict(
                kbits=kb, vbits=vb, cap=cap,
                kq=np.zeros((B, Hkv, kb // 2, cap, D // 16), np.uint32),
                ks=np.zeros((B, Hkv, cap // Gk, D), np.uint16),
                kz=np.zeros((B, Hkv, cap // Gk, D), np.uint16),
                vq=np.zeros((B, Hkv, vb // 2, cap // 16, D), np.uint32),
                vs=np.zeros((B, Hkv, cap, D // Gv), np.uint16),
                vz=np.zeros((B, Hkv, cap, D // Gv), np.uint16),
                n=np.zeros((B, Hkv), np.int64)))
        self.kres = np.zeros((B, Hkv, residual_cap, D), np.uint16)
        self.vres = np.zeros_like(self.kres)
        self.n_res = 0

    def _store(self, si, b, h, at, out):
        S, Gk = self.segs[si], self.Gk
        mp = out["kq"].shape[1]
        if at + mp > S["cap"]:
            raise ValueError("capacity exceeded")
        S["kq"][b, h, :, at:at + mp] = out["kq"]
        S["ks"][b, h, at // Gk:(at + mp) // Gk] = out["ks"]
        S["kz"][b, h, at // Gk:(at + mp) // Gk] = out["kz"]
        S["vq"][b, h, :, at // 16:(at + mp) // 16] = out["vq"]
        S["vs"][b, h, at:at + mp] = out["vs"]
        S["vz"][b, h, at:at + mp] = out["vz"]
        S["n"][b, h] = at + mp

    def pack(self, si, k, v, b, h, idx, tail=True):
        """Pack token indices idx (ascending) of unit (b, h) into segment si
        (replacing its contents); with tail, the last len(idx) mod Gk go to
        the end of the residual."""
        S = self.segs[si]
        out = pack_unit_bits(_u16(k)[b, h], _u16(v)[b, h], idx, self.Gk,
                             self.Gv, S["kbits"], S["vbits"])
        self._store(si, b, h, 0, out)
        t = out["kres"].shape[0]
        assert tail or t == 0
        return out["kres"], out["vres"]

    def set_residual(self, kres, vres):
        """kres, vres [B][Hkv][t][D], the same t for every unit."""
        t = kres.shape[2]
        assert t < self.nr
        self.kres[:, :, :t] = _u16(kres)
        self.vres[:, :, :t] = _u16(vres)
        self.n_res = t

    def append(self, k_new, v_new):
        k_new, v_new = _u16(k_new), _u16(v_new)
        S = self.segs[self.flush_seg]
        if self.n_res + 1 == self.nr and S["n"].max() + self.nr > S["cap"]:
            raise ValueError("capacity exceeded")
        self.kres[:, :, self.n_res] = k_new
        self.vres[:, :, self.n_res] = v_new
        self.n_res += 1
        if self.n_res == self.nr:
            ident = np.arange(self.nr, dtype=np.int32)
            for b in range(self.B):
                for h in range(self.Hkv):
                    out = pack_unit_bits(self.kres[b, h], self.vres[b, h], ident,
                                         self.Gk, self.Gv, S["kbits"],
                                         S["vbits"])
                    self._store(self.flush_seg, b, h, int(S["n"][b, h]), out)
            self.n_res = 0

    def decode_unit(self, qg, b, h):
        """o [g][D] fp64: attention over every segment's packed tokens of
        unit (b, h) and the residual (order does not matter)."""
        ks_, vs_ = [], []
        for S in self.segs:
            kh, vh = dequant_unit(self.Gk, self.Gv, S["kbits"], S["vbits"],
                                  int(S["n"][b, h]), S["kq"][b, h], S["ks"][b, h],
                                  S["kz"][b, h], S["vq"][b, h], S["vs"][b, h],
                                  S["vz"][b, h])
            ks_.append(kh)
            vs_.append(vh)
        r = self.n_res
        ks_.append(np.vectorize(h2d)(self.kres[b, h, :r]).reshape(r, self.D)
                   if r else np.zeros((0, self.D)))
        vs_.append(np.vectorize(h2d)(self.vres[b, h, :r]).reshape(r, self.D)
                   if r else np.zeros((0, self.D)))
        return attend(qg, np.concatenate(ks_), np.concatenate(vs_))
