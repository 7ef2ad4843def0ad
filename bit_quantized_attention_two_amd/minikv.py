"""ctypes binding of libminikv.so (include/minikv.h).

Argument marshalling only: torch tensors supply device memory and the
current HIP stream; every step of the computation runs in the library's HIP
kernels.  The binding refuses to work without the built library -- there is
no fallback path.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libminikv.so")

OK, EINVAL, EUNSUPPORTED, ECAPACITY, EHIP = 0, -1, -2, -3, -4

_i32 = ctypes.c_int32
_P = ctypes.c_void_p
_sz = ctypes.c_size_t


class MiniKVError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("%s: %s" % (status_str(status) if _lib else status,
                                     msg))
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("batch", _i32), ("n_q_heads", _i32), ("n_kv_heads", _i32),
                ("head_dim", _i32), ("group_k", _i32), ("group_v", _i32),
                ("residual_cap", _i32)]

    @property
    def units(self):
        return self.batch * self.n_kv_heads

    @property
    def g(self):
        return self.n_q_heads // self.n_kv_heads


class _CacheC(ctypes.Structure):
    _fields_ = [("kq", _P), ("k_scale", _P), ("k_zero", _P), ("vq", _P),
                ("v_scale", _P), ("v_zero", _P), ("k_res", _P), ("v_res", _P),
                ("capacity", _i32), ("n_packed", _i32), ("n_res", _i32)]


_lib = None


def lib():
    """Load libminikv.so (build it first: python -m
    bit_quantized_attention_two_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libminikv.so is not built (%s); run "
                               "`python -m bit_quantized_attention_two_amd."
                               "build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        D = ctypes.POINTER(Dims)
        C = ctypes.POINTER(_CacheC)
        sig = {
            "minikv_version": ([], _i32),
            "minikv_status_str": ([_i32], ctypes.c_char_p),
            "minikv_last_error": ([], ctypes.c_char_p),
            "minikv_pyramid_budgets": ([_i32] * 8 + [_P, _P], _i32),
            "minikv_cache_bytes_closed_form": ([_i32] * 9 + [_P, _P], _i32),
            "minikv_cache_layout": ([D, _i32, _P], _i32),
            "minikv_prefill_ws_bytes": ([D, _i32, _i32, _P], _i32),
            "minikv_decode_ws_bytes": ([D, _i32, _P], _i32),
            "minikv_decode_mass_ws_bytes": ([D, _i32, _P], _i32),
            "minikv_prefill_attn": ([D, _i32, _P, _P, _P, _P, _P, _P, _P],
                                    _i32),
            "minikv_select": ([D, _i32, _P, _i32, _i32, _P, _P], _i32),
            "minikv_prefill_select": ([D, _i32, _P, _P, _P, _P, _P, _P, _i32,
                                       _i32, _P, _P, _sz, _P], _i32),
            "minikv_pack": ([D, _i32, _P, _P, _P, _i32, C, _P], _i32),
            "minikv_append": ([D, C, _P, _P, _P], _i32),
            "minikv_decode_attn": ([D, C, _P, _P, _P, _sz, _P], _i32),
            "minikv_decode_attn_mass": ([D, C, _P, _P, _P, _i32, _P, _sz, _P],
                                        _i32),
            "minikv_append_decode": ([D, C, _P, _P, _P, _P, _P, _sz, _P],
                                     _i32),
            "minikv_decode_attn_noalloc": ([D, C, _P, _P, _P], _i32),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


EXPORTED = ("minikv_version", "minikv_status_str", "minikv_last_error",
            "minikv_pyramid_budgets", "minikv_cache_bytes_closed_form",
            "minikv_cache_layout", "minikv_prefill_ws_bytes",
            "minikv_decode_ws_bytes", "minikv_prefill_attn", "minikv_select",
            "minikv_prefill_select", "minikv_pack", "minikv_append",
            "minikv_decode_attn", "minikv_append_decode",
            "minikv_decode_mass_ws_bytes", "minikv_decode_attn_mass",
            "minikv_decode_attn_noalloc")


def status_str(s):
    return lib().minikv_status_str(s).decode()


def _check(status):
    if status != OK:
        raise MiniKVError(status, lib().minikv_last_error().decode())


def _ptr(t):
    return None if t is None else _P(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return _P(stream.cuda_stream)


def _on_device(t):
    return t.is_cuda


def _need(t, dtype, shape, name):
    """Every tensor handed to the library -- inputs and caller-supplied
    outputs alike -- must have exactly the dtype, shape and contiguity the
    kernels read or write: the C ABI cannot see buffer sizes, so a wrong
    output would be written out of bounds."""
    if not hasattr(t, "dtype") or t.dtype != dtype or \
            tuple(t.shape) != tuple(shape) or not t.is_contiguous() or \
            not _on_device(t):
        raise ValueError("%s must be a contiguous CUDA %s tensor of shape %s "
                         "(got %s)" % (name, dtype, tuple(shape),
                                       "%s %s" % (t.dtype, tuple(t.shape))
                                       if hasattr(t, "dtype") else type(t)))


def _out(t, dtype, shape, name, like):
    """A caller-supplied output, checked, or a new one on like's device."""
    if t is None:
        return torch.empty(shape, dtype=dtype, device=like.device)
    _need(t, dtype, shape, name)
    return t


def _ws(t, nbytes, name="ws"):
    """A caller-supplied workspace: contiguous device bytes, at least
    nbytes (the library checks the size it is told against its need)."""
    if not hasattr(t, "is_contiguous") or not t.is_contiguous() or \
            not _on_device(t) or t.numel() * t.element_size() < nbytes:
        raise ValueError("%s must be a contiguous CUDA buffer of at least %d "
                         "bytes" % (name, nbytes))
    return t.numel() * t.element_size()


def make_dims(B, Hq, Hkv, D, Gk=16, Gv=16, residual_cap=128):
    return Dims(B, Hq, Hkv, D, Gk, Gv, residual_cap)


# ----------------------------------------------------------- host helpers --

def pyramid_budgets(n, n_layers, hh=(1, 4), rw=(1, 4), depth=7,
                    pyramid=True):
    k = (ctypes.c_int32 * n_layers)()
    r = ctypes.c_int32()
    _check(lib().minikv_pyramid_budgets(n, n_layers, hh[0], hh[1], rw[0],
                                        rw[1], depth, 1 if pyramid else 0,
                                        ctypes.cast(k, _P),
                                        ctypes.cast(ctypes.pointer(r), _P)))
    return list(k), r.value


def cache_bytes_closed_form(n_layers, n_heads, head_dim, lprompt, lgen,
                            budget=(1, 2), bits=2, group=16):
    a, b = ctypes.c_uint64(), ctypes.c_uint64()
    _check(lib().minikv_cache_bytes_closed_form(
        n_layers, n_heads, head_dim, lprompt, lgen, budget[0], budget[1],
        bits, group, ctypes.cast(ctypes.pointer(a), _P),
        ctypes.cast(ctypes.pointer(b), _P)))
    return a.value, b.value


def cache_layout(dims, capacity):
    out = (ctypes.c_size_t * 8)()
    _check(lib().minikv_cache_layout(ctypes.byref(dims), capacity,
                                     ctypes.cast(out, _P)))
    return list(out)


def prefill_ws_bytes(dims, n, lse_given=False):
    out = ctypes.c_size_t()
    _check(lib().minikv_prefill_ws_bytes(ctypes.byref(dims), n,
                                         1 if lse_given else 0,
                                         ctypes.cast(ctypes.pointer(out), _P)))
    return out.value


def decode_ws_bytes(dims, capacity):
    out = ctypes.c_size_t()
    _check(lib().minikv_decode_ws_bytes(ctypes.byref(dims), capacity,
                                        ctypes.cast(ctypes.pointer(out), _P)))
    return out.value


# ----------------------------------------------------------------- caches --

class LayerCache:
    """Device arrays of one layer's compressed cache plus the host counters
    (layout in include/minikv.h)."""

    NAMES = ("kq", "k_scale", "k_zero", "vq", "v_scale", "v_zero", "k_res",
             "v_res")

    def __init__(self, dims, capacity, device="cuda"):
        self.dims = dims
        sizes = cache_layout(dims, capacity)
        U, D = dims.units, dims.head_dim
        Gk, Gv, nr = dims.group_k, dims.group_v, dims.residual_cap
        shapes = {
            "kq": ((U, capacity, D // 16), torch.int32),
            "k_scale": ((U, capacity // Gk, D), torch.float16),
            "k_zero": ((U, capacity // Gk, D), torch.float16),
            "vq": ((U, capacity // 16, D), torch.int32),
            "v_scale": ((U, capacity, D // Gv), torch.float16),
            "v_zero": ((U, capacity, D // Gv), torch.float16),
            "k_res": ((U, nr, D), torch.float16),
            "v_res": ((U, nr, D), torch.float16),
        }
        for name, nbytes in zip(self.NAMES, sizes):
            shape, dt = shapes[name]
            t = torch.zeros(shape, dtype=dt, device=device)
            assert t.numel() * t.element_size() == nbytes
            setattr(self, name, t)
        self.c = _CacheC(*[_P(getattr(self, n).data_ptr()) for n in self.NAMES],
                         capacity, 0, 0)

    @property
    def capacity(self):
        return self.c.capacity

    @property
    def n_packed(self):
        return self.c.n_packed

    @property
    def n_res(self):
        return self.c.n_res

    def nbytes(self):
        return sum(getattr(self, n).numel() * getattr(self, n).element_size()
                   for n in self.NAMES)


# ---------------------------------------------------------- compute calls --

def prefill_attn(dims, q, k, v, o=None, lse=None, col=None, stream=None):
    B, Hq, Hkv, D = dims.batch, dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    n = q.shape[2]
    _need(q, torch.float16, (B, Hq, n, D), "q")
    _need(k, torch.float16, (B, Hkv, n, D), "k")
    _need(v, torch.float16, (B, Hkv, n, D), "v")
    o = _out(o, torch.float16, (B, Hq, n, D), "o", q)
    lse = _out(lse, torch.float32, (B, Hq, n), "lse", q)
    col = _out(col, torch.float32, (B, Hkv, n), "col", q)
    _check(lib().minikv_prefill_attn(ctypes.byref(dims), n, _ptr(q), _ptr(k),
                                     _ptr(v), _ptr(o), _ptr(lse), _ptr(col),
                                     _stream(stream)))
    return o, lse, col


def select(dims, col, n_hh, n_recent, sel=None, stream=None):
    B, Hkv = dims.batch, dims.n_kv_heads
    n = col.shape[-1]
    _need(col, torch.float32, (B, Hkv, n), "col")
    sel = _out(sel, torch.int32, (B, Hkv, n_hh + n_recent), "sel", col)
    _check(lib().minikv_select(ctypes.byref(dims), n, _ptr(col), n_hh,
                               n_recent, _ptr(sel), _stream(stream)))
    return sel


def prefill_select(dims, q, k, v, n_hh, n_recent, o=None, col=None, lse=None,
                   sel=None, ws=None, stream=None):
    B, Hq, Hkv, D = dims.batch, dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    n = q.shape[2]
    _need(q, torch.float16, (B, Hq, n, D), "q")
    _need(k, torch.float16, (B, Hkv, n, D), "k")
    _need(v, torch.float16, (B, Hkv, n, D), "v")
    o = _out(o, torch.float16, (B, Hq, n, D), "o", q)
    col = _out(col, torch.float32, (B, Hkv, n), "col", q)
    sel = _out(sel, torch.int32, (B, Hkv, n_hh + n_recent), "sel", q)
    if lse is not None:
        _need(lse, torch.float32, (B, Hq, n), "lse")
    ws_bytes = 0
    if lse is None and ws is None:
        ws = torch.empty(prefill_ws_bytes(dims, n), dtype=torch.uint8,
                         device=q.device)
    if ws is not None:
        ws_bytes = _ws(ws, 0 if lse is not None else prefill_ws_bytes(dims, n))
    _check(lib().minikv_prefill_select(
        ctypes.byref(dims), n, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(col),
        _ptr(lse), n_hh, n_recent, _ptr(sel), _ptr(ws), ws_bytes,
        _stream(stream)))
    return o, col, sel


def pack(dims, k, v, sel, cache, stream=None):
    B, Hkv, D = dims.batch, dims.n_kv_heads, dims.head_dim
    n = k.shape[2]
    _need(k, torch.float16, (B, Hkv, n, D), "k")
    _need(v, torch.float16, (B, Hkv, n, D), "v")
    n_sel = sel.shape[-1]
    _need(sel, torch.int32, (B, Hkv, n_sel), "sel")
    _check(lib().minikv_pack(ctypes.byref(dims), n, _ptr(k), _ptr(v),
                             _ptr(sel), n_sel, ctypes.byref(cache.c),
                             _stream(stream)))


def append(dims, cache, k_new, v_new, stream=None):
    shape = (dims.batch, dims.n_kv_heads, dims.head_dim)
    _need(k_new, torch.float16, shape, "k_new")
    _need(v_new, torch.float16, shape, "v_new")
    _check(lib().minikv_append(ctypes.byref(dims), ctypes.byref(cache.c),
                               _ptr(k_new), _ptr(v_new), _stream(stream)))


def decode_mass_ws_bytes(dims, capacity):
    out = ctypes.c_size_t()
    _check(lib().minikv_decode_mass_ws_bytes(
        ctypes.byref(dims), capacity, ctypes.cast(ctypes.pointer(out), _P)))
    return out.value


def decode_attn_mass(dims, cache, q, mass, o=None, ws=None, stream=None):
    """decode_attn(q), and mass[b, kvh, t] += the attention weight of cache
    token t summed over the kv head's query heads (persistence audit).
    mass: fp32 [B][Hkv][stride], stride >= n_packed + n_res."""
    shape = (dims.batch, dims.n_q_heads, dims.head_dim)
    _need(q, torch.float16, shape, "q")
    if (mass.dtype != torch.float32 or mass.dim() != 3 or not mass.is_contiguous()
            or not _on_device(mass)
            or tuple(mass.shape[:2]) != (dims.batch, dims.n_kv_heads)):
        raise ValueError("mass: contiguous fp32 [B][Hkv][stride] expected")
    o = _out(o, torch.float16, shape, "o", q)
    need = decode_mass_ws_bytes(dims, cache.capacity)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = _ws(ws, need)
    _check(lib().minikv_decode_attn_mass(
        ctypes.byref(dims), ctypes.byref(cache.c), _ptr(q), _ptr(o),
        _ptr(mass), mass.shape[2], _ptr(ws), ws_bytes, _stream(stream)))
    return o


def decode_attn(dims, cache, q, o=None, ws=None, stream=None):
    shape = (dims.batch, dims.n_q_heads, dims.head_dim)
    _need(q, torch.float16, shape, "q")
    o = _out(o, torch.float16, shape, "o", q)
    need = decode_ws_bytes(dims, cache.capacity)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = _ws(ws, need)
    _check(lib().minikv_decode_attn(ctypes.byref(dims), ctypes.byref(cache.c),
                                    _ptr(q), _ptr(o), _ptr(ws), ws_bytes,
                                    _stream(stream)))
    return o


def append_decode(dims, cache, k_new, v_new, q, o=None, ws=None, stream=None):
    """append(k_new, v_new) then decode_attn(q), fused when no flush is due."""
    kshape = (dims.batch, dims.n_kv_heads, dims.head_dim)
    _need(k_new, torch.float16, kshape, "k_new")
    _need(v_new, torch.float16, kshape, "v_new")
    _need(q, torch.float16, (dims.batch, dims.n_q_heads, dims.head_dim), "q")
    o = _out(o, torch.float16, (dims.batch, dims.n_q_heads, dims.head_dim),
             "o", q)
    need = decode_ws_bytes(dims, cache.capacity)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = _ws(ws, need)
    _check(lib().minikv_append_decode(
        ctypes.byref(dims), ctypes.byref(cache.c), _ptr(k_new), _ptr(v_new),
        _ptr(q), _ptr(o), _ptr(ws), ws_bytes, _stream(stream)))
    return o


def decode_attn_noalloc(dims, cache, q, o=None, stream=None):
    """decode_attn without a workspace: the library's own per-device scratch
    array holds the split partials (calls on one GPU must not overlap)."""
    shape = (dims.batch, dims.n_q_heads, dims.head_dim)
    _need(q, torch.float16, shape, "q")
    o = _out(o, torch.float16, shape, "o", q)
    _check(lib().minikv_decode_attn_noalloc(ctypes.byref(dims),
                                            ctypes.byref(cache.c), _ptr(q),
                                            _ptr(o), _stream(stream)))
    return o


# ------------------------------------------------ mixed-precision caches --
# MiKV (important tokens at high precision, the rest kept at low precision)
# and DiffKV (K8V4 / K4V2 tiers by significance, pruning the rest): packed
# segments of their own bit widths plus one fp16 residual
# (include/minikv.h, "mixed-precision caches").

MAX_SEGMENTS = 3


class _SegC(ctypes.Structure):
    _fields_ = [("kq", _P), ("k_scale", _P), ("k_zero", _P), ("vq", _P),
                ("v_scale", _P), ("v_zero", _P), ("key_bits", _i32),
                ("value_bits", _i32), ("capacity", _i32), ("n_packed", _i32),
                ("n_unit", _P)]


class _MixedC(ctypes.Structure):
    _fields_ = [("seg", _SegC * MAX_SEGMENTS), ("n_seg", _i32),
                ("flush_seg", _i32), ("k_res", _P), ("v_res", _P),
                ("n_res", _i32)]


_MIXED_SIG = {
    "minikv_segment_layout": (["D", _i32, _i32, _i32, _P], _i32),
    "minikv_mikv_ws_bytes": (["D", _i32, _i32, _P], _i32),
    "minikv_pack_mikv": (["D", _i32, _P, _P, _P, _i32, "M", _P, _sz, _P], _i32),
    "minikv_append_mixed": (["D", "M", _P, _P, _P], _i32),
    "minikv_decode_mixed_ws_bytes": (["D", "M", _P], _i32),
    "minikv_decode_mixed": (["D", "M", _P, _P, _P, _sz, _P], _i32),
    "minikv_diffkv_ws_bytes": (["D", _i32, _i32, _P], _i32),
    "minikv_prefill_diffkv": (["D", _i32, _P, _P, _P, _P, _P, _P, _P, _sz, _P],
                              _i32),
    "minikv_tier_diffkv": (["D", _i32, _P, ctypes.c_float, ctypes.c_float, _P,
                           _P, _P, _P, _P], _i32),
    "minikv_pack_diffkv": (["D", _i32, _P, _P, _P, _P, _P, _P, "M", _P], _i32),
}
EXPORTED = EXPORTED + tuple(_MIXED_SIG)


def _mixed_lib():
    L = lib()
    if not getattr(L, "_mixed_sig_set", False):
        D = ctypes.POINTER(Dims)
        M = ctypes.POINTER(_MixedC)
        for name, (args, res) in _MIXED_SIG.items():
            f = getattr(L, name)
            f.argtypes = [D if a == "D" else M if a == "M" else a for a in args]
            f.restype = res
        L._mixed_sig_set = True
    return L


def segment_layout(dims, key_bits, value_bits, capacity):
    out = (ctypes.c_size_t * 6)()
    _check(_mixed_lib().minikv_segment_layout(ctypes.byref(dims), key_bits,
                                              value_bits, capacity,
                                              ctypes.cast(out, _P)))
    return list(out)


class MixedCache:
    """Device arrays of a mixed-precision cache: `segs` is a list of
    (key_bits, value_bits, capacity); flush_seg receives residual flushes.
    Segment i's arrays are self.seg[i][name] with
      kq [U][key_bits/2][cap][D/16] int32, k_scale/k_zero [U][cap/Gk][D],
      vq [U][value_bits/2][cap/16][D] int32, v_scale/v_zero [U][cap][D/Gv]."""

    SEG_NAMES = ("kq", "k_scale", "k_zero", "vq", "v_scale", "v_zero")

    def __init__(self, dims, segs, flush_seg=0, device="cuda"):
        assert 1 <= len(segs) <= MAX_SEGMENTS
        self.dims = dims
        U, D = dims.units, dims.head_dim
        Gk, Gv, nr = dims.group_k, dims.group_v, dims.residual_cap
        self.c = _MixedC()
        self.seg = []
        for i, (kb, vb, cap) in enumerate(segs):
            sizes = segment_layout(dims, kb, vb, cap)
            shapes = {
                "kq": ((U, kb // 2, cap, D // 16), torch.int32),
                "k_scale": ((U, cap // Gk, D), torch.float16),
                "k_zero": ((U, cap // Gk, D), torch.float16),
                "vq": ((U, vb // 2, cap // 16, D), torch.int32),
                "v_scale": ((U, cap, D // Gv), torch.float16),
                "v_zero": ((U, cap, D // Gv), torch.float16),
            }
            arrs = {}
            for name, nbytes in zip(self.SEG_NAMES, sizes):
                shape, dt = shapes[name]
                t = torch.zeros(shape, dtype=dt, device=device)
                assert t.numel() * t.element_size() == nbytes
                arrs[name] = t
            self.seg.append(arrs)
            s = self.c.seg[i]
            for name in self.SEG_NAMES:
                setattr(s, name, _P(arrs[name].data_ptr()))
            s.key_bits, s.value_bits, s.capacity, s.n_packed = kb, vb, cap, 0
            s.n_unit = None
        self.c.n_seg = len(segs)
        self.c.flush_seg = flush_seg
        self.k_res = torch.zeros((U, nr, D), dtype=torch.float16, device=device)
        self.v_res = torch.zeros_like(self.k_res)
        self.c.k_res = _P(self.k_res.data_ptr())
        self.c.v_res = _P(self.v_res.data_ptr())
        self.c.n_res = 0
        self._keep = []                      # device count arrays in use

    @property
    def n_res(self):
        return self.c.n_res

    def n_packed(self, i):
        return self.c.seg[i].n_packed

    def set_bound(self, i, bound):
        """Lower segment i's packed-token bound (e.g. to the largest
        per-unit count after reading the counts back)."""
        self.c.seg[i].n_packed = int(bound)

    def nbytes(self):
        return sum(t.numel() * t.element_size() for s in self.seg for t in s.values()) + \
            2 * self.k_res.numel() * 2


def mikv_ws_bytes(dims, n, n_sel):
    out = ctypes.c_size_t()
    _check(_mixed_lib().minikv_mikv_ws_bytes(ctypes.byref(dims), n, n_sel,
                                             ctypes.cast(ctypes.pointer(out), _P)))
    return out.value


def pack_mikv(dims, k, v, sel, cache, ws=None, stream=None):
    """MiKV pack: sel (the important tokens) into segment 0, the other
    tokens into segment 1, tails to the fp16 residual."""
    B, Hkv, D = dims.batch, dims.n_kv_heads, dims.head_dim
    n = k.shape[2]
    _need(k, torch.float16, (B, Hkv, n, D), "k")
    _need(v, torch.float16, (B, Hkv, n, D), "v")
    n_sel = sel.shape[-1]
    _need(sel, torch.int32, (B, Hkv, n_sel), "sel")
    need = mikv_ws_bytes(dims, n, n_sel)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=k.device)
    ws_bytes = _ws(ws, need)
    _check(_mixed_lib().minikv_pack_mikv(
        ctypes.byref(dims), n, _ptr(k), _ptr(v), _ptr(sel), n_sel,
        ctypes.byref(cache.c), _ptr(ws), ws_bytes, _stream(stream)))


def append_mixed(dims, cache, k_new, v_new, stream=None):
    shape = (dims.batch, dims.n_kv_heads, dims.head_dim)
    _need(k_new, torch.float16, shape, "k_new")
    _need(v_new, torch.float16, shape, "v_new")
    _check(_mixed_lib().minikv_append_mixed(ctypes.byref(dims),
                                            ctypes.byref(cache.c), _ptr(k_new),
                                            _ptr(v_new), _stream(stream)))


def decode_mixed_ws_bytes(dims, cache):
    out = ctypes.c_size_t()
    _check(_mixed_lib().minikv_decode_mixed_ws_bytes(
        ctypes.byref(dims), ctypes.byref(cache.c),
        ctypes.cast(ctypes.pointer(out), _P)))
    return out.value


def decode_mixed(dims, cache, q, o=None, ws=None, stream=None):
    shape = (dims.batch, dims.n_q_heads, dims.head_dim)
    _need(q, torch.float16, shape, "q")
    o = _out(o, torch.float16, shape, "o", q)
    need = decode_mixed_ws_bytes(dims, cache)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = _ws(ws, need)
    _check(_mixed_lib().minikv_decode_mixed(ctypes.byref(dims),
                                            ctypes.byref(cache.c), _ptr(q),
                                            _ptr(o), _ptr(ws), ws_bytes,
                                            _stream(stream)))
    return o


def prefill_diffkv(dims, q, k, v, o=None, score=None, lse=None, ws=None,
                   stream=None):
    """Prefill attention plus DiffKV's per-key significance [B][Hkv][n]."""
    B, Hq, Hkv, D = dims.batch, dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    n = q.shape[2]
    _need(q, torch.float16, (B, Hq, n, D), "q")
    _need(k, torch.float16, (B, Hkv, n, D), "k")
    _need(v, torch.float16, (B, Hkv, n, D), "v")
    o = _out(o, torch.float16, (B, Hq, n, D), "o", q)
    score = _out(score, torch.float32, (B, Hkv, n), "score", q)
    ws_bytes = 0
    if lse is not None:
        _need(lse, torch.float32, (B, Hq, n), "lse")
    elif ws is None:
        ws = torch.empty(prefill_ws_bytes(dims, n), dtype=torch.uint8,
                         device=q.device)
    if ws is not None:
        ws_bytes = _ws(ws, 0 if lse is not None else prefill_ws_bytes(dims, n))
    _check(_mixed_lib().minikv_prefill_diffkv(
        ctypes.byref(dims), n, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(score),
        _ptr(lse), _ptr(ws), ws_bytes, _stream(stream)))
    return o, score


def tier_diffkv(dims, score, alpha_hi, alpha_lo, idx_hi=None, idx_lo=None,
                n_hi=None, n_lo=None, stream=None):
    """DiffKV tiers: (idx_hi, idx_lo [B][Hkv][n], n_hi, n_lo [B*Hkv])."""
    B, Hkv = dims.batch, dims.n_kv_heads
    n = score.shape[-1]
    _need(score, torch.float32, (B, Hkv, n), "score")
    idx_hi = _out(idx_hi, torch.int32, (B, Hkv, n), "idx_hi", score)
    idx_lo = _out(idx_lo, torch.int32, (B, Hkv, n), "idx_lo", score)
    n_hi = _out(n_hi, torch.int32, (B * Hkv,), "n_hi", score)
    n_lo = _out(n_lo, torch.int32, (B * Hkv,), "n_lo", score)
    _check(_mixed_lib().minikv_tier_diffkv(
        ctypes.byref(dims), n, _ptr(score), float(alpha_hi), float(alpha_lo),
        _ptr(idx_hi), _ptr(idx_lo), _ptr(n_hi), _ptr(n_lo), _stream(stream)))
    return idx_hi, idx_lo, n_hi, n_lo


def pack_diffkv(dims, k, v, idx_hi, idx_lo, n_hi, n_lo, cache, stream=None):
    """DiffKV pack into a three-segment cache (K8V4 tier, K4V2 tier,
    generated tokens at K8V4); the count arrays stay referenced by the
    cache."""
    B, Hkv, D = dims.batch, dims.n_kv_heads, dims.head_dim
    n = k.shape[2]
    _need(k, torch.float16, (B, Hkv, n, D), "k")
    _need(v, torch.float16, (B, Hkv, n, D), "v")
    for t, name in ((idx_hi, "idx_hi"), (idx_lo, "idx_lo")):
        _need(t, torch.int32, (B, Hkv, n), name)
    for t, name in ((n_hi, "n_hi"), (n_lo, "n_lo")):
        _need(t, torch.int32, (B * Hkv,), name)
    _check(_mixed_lib().minikv_pack_diffkv(
        ctypes.byref(dims), n, _ptr(k), _ptr(v), _ptr(idx_hi), _ptr(idx_lo),
        _ptr(n_hi), _ptr(n_lo), ctypes.byref(cache.c), _stream(stream)))
    cache._keep = [n_hi, n_lo]


# ------------------------------------------------------ fused prefill tail --

_TAIL_SIG = {
    "minikv_prefill_tail_ws_bytes": (["D", _i32, _i32, _P], _i32),
    "minikv_prefill_select_pack": (["D", _i32, _P, _P, _P, _P, _P, _P, _i32, _i32,
                                    _P, "C", _i32, _P, _sz, _P], _i32),
}
EXPORTED = EXPORTED + tuple(_TAIL_SIG)


def _tail_lib():
    L = lib()
    if not getattr(L, "_tail_sig_set", False):
        D = ctypes.POINTER(Dims)
        C = ctypes.POINTER(_CacheC)
        for name, (args, res) in _TAIL_SIG.items():
            f = getattr(L, name)
            f.argtypes = [D if a == "D" else C if a == "C" else a for a in args]
            f.restype = res
        L._tail_sig_set = True
    return L


def prefill_tail_ws_bytes(dims, n, lse_given=False):
    out = ctypes.c_size_t()
    _check(_tail_lib().minikv_prefill_tail_ws_bytes(
        ctypes.byref(dims), n, 1 if lse_given else 0,
        ctypes.cast(ctypes.pointer(out), _P)))
    return out.value


def prefill_select_pack(dims, q, k, v, n_hh, n_recent, cache, fuse_select=False,
                        o=None, col=None, lse=None, sel=None, ws=None,
                        stream=None):
    """prefill_select then pack in one call, the selection fused into the
    second prefill pass when fuse_select; returns (o, col, sel)."""
    B, Hq, Hkv, D = dims.batch, dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    n = q.shape[2]
    _need(q, torch.float16, (B, Hq, n, D), "q")
    _need(k, torch.float16, (B, Hkv, n, D), "k")
    _need(v, torch.float16, (B, Hkv, n, D), "v")
    o = _out(o, torch.float16, (B, Hq, n, D), "o", q)
    col = _out(col, torch.float32, (B, Hkv, n), "col", q)
    sel = _out(sel, torch.int32, (B, Hkv, n_hh + n_recent), "sel", q)
    if lse is not None:
        _need(lse, torch.float32, (B, Hq, n), "lse")
    need = prefill_tail_ws_bytes(dims, n, lse is not None)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = _ws(ws, need)
    _check(_tail_lib().minikv_prefill_select_pack(
        ctypes.byref(dims), n, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(col),
        _ptr(lse), n_hh, n_recent, _ptr(sel), ctypes.byref(cache.c),
        1 if fuse_select else 0, _ptr(ws), ws_bytes, _stream(stream)))
    return o, col, sel
