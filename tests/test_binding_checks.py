"""CPU checks of the Python binding: every caller-supplied output and
workspace is checked for dtype, shape and contiguity before any compute call
reaches the library (the C ABI cannot see buffer sizes, so a wrong output
would be written out of bounds).  The library is wrapped so that reaching a
compute entry point fails the test; CPU tensors stand in for device tensors.
"""
import pytest
import torch

COMPUTE = {"minikv_prefill_attn", "minikv_select", "minikv_prefill_select",
           "minikv_pack", "minikv_append", "minikv_decode_attn",
           "minikv_append_decode", "minikv_decode_attn_mass",
           "minikv_decode_attn_noalloc"}


class Launched(Exception):
    pass


class _Guard:
    def __init__(self, real):
        self.real = real

    def __getattr__(self, name):
        if name in COMPUTE:
            raise Launched(name)
        return getattr(self.real, name)


@pytest.fixture
def mk(monkeypatch):
    from bit_quantized_attention_two_amd import minikv
    import os
    if not os.path.exists(minikv.LIB_PATH):
        from bit_quantized_attention_two_amd import build
        build.build()
    monkeypatch.setattr(minikv, "_lib", _Guard(minikv.lib()))
    monkeypatch.setattr(minikv, "_on_device", lambda t: True)
    return minikv


def _h(*shape):
    return torch.zeros(shape, dtype=torch.float16)


def test_prefill_outputs_checked(mk):
    B, Hq, Hkv, n, D = 1, 4, 2, 64, 64
    dims = mk.make_dims(B, Hq, Hkv, D)
    q, k, v = _h(B, Hq, n, D), _h(B, Hkv, n, D), _h(B, Hkv, n, D)
    bad = [
        dict(o=_h(B, Hq, n - 1, D)),
        dict(o=torch.zeros((B, Hq, n, D), dtype=torch.float32)),
        dict(o=_h(B, Hq, D, n).transpose(2, 3)),          # not contiguous
        dict(lse=torch.zeros((B, Hq, n + 1))),
        dict(lse=torch.zeros((B, Hq, n), dtype=torch.float16)),
        dict(col=torch.zeros((B, Hq, n))),                  # per q head
    ]
    for kw in bad:
        with pytest.raises(ValueError):
            mk.prefill_attn(dims, q, k, v, **kw)
    with pytest.raises(Launched):                           # control
        mk.prefill_attn(dims, q, k, v)


def test_prefill_select_outputs_checked(mk):
    B, Hq, Hkv, n, D = 2, 4, 4, 64, 128
    dims = mk.make_dims(B, Hq, Hkv, D)
    q, k, v = _h(B, Hq, n, D), _h(B, Hkv, n, D), _h(B, Hkv, n, D)
    bad = [
        dict(sel=torch.zeros((B, Hkv, 31), dtype=torch.int32)),
        dict(sel=torch.zeros((B, Hkv, 32), dtype=torch.int64)),
        dict(col=torch.zeros((B, Hkv, n - 16))),
        dict(o=_h(B, Hq, n, 64)),
        dict(lse=torch.zeros((B, Hq, n + 1))),
        dict(ws=torch.zeros(16, dtype=torch.uint8)),        # too small
    ]
    for kw in bad:
        with pytest.raises(ValueError):
            mk.prefill_select(dims, q, k, v, 16, 16, **kw)
    with pytest.raises(Launched):
        mk.prefill_select(dims, q, k, v, 16, 16)


def test_select_output_checked(mk):
    dims = mk.make_dims(1, 2, 2, 128)
    col = torch.zeros((1, 2, 100))
    with pytest.raises(ValueError):
        mk.select(dims, col, 10, 10, sel=torch.zeros((1, 2, 21), dtype=torch.int32))
    with pytest.raises(ValueError):
        mk.select(dims, col, 10, 10, sel=torch.zeros((2, 1, 20), dtype=torch.int32))
    with pytest.raises(Launched):
        mk.select(dims, col, 10, 10)


def test_decode_outputs_checked(mk):
    B, Hq, Hkv, D = 2, 8, 2, 128
    dims = mk.make_dims(B, Hq, Hkv, D)
    cache = mk.LayerCache(dims, 64, device="cpu")
    q = _h(B, Hq, D)
    kn = _h(B, Hkv, D)
    for kw in (dict(o=_h(B, Hkv, D)), dict(o=_h(B, Hq, D + 1)),
               dict(o=torch.zeros((B, Hq, D))),
               dict(ws=torch.zeros(8, dtype=torch.uint8))):
        with pytest.raises(ValueError):
            mk.decode_attn(dims, cache, q, **kw)
        with pytest.raises(ValueError):
            mk.append_decode(dims, cache, kn, kn, q, **kw)
    mass = torch.zeros((B, Hkv, 256))
    with pytest.raises(ValueError):
        mk.decode_attn_mass(dims, cache, q, mass, o=_h(B, Hq, 64))
    with pytest.raises(ValueError):
        mk.decode_attn_mass(dims, cache, q, torch.zeros((B, Hq, 256)))
    with pytest.raises(Launched):
        mk.decode_attn(dims, cache, q)
