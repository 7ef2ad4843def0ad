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
