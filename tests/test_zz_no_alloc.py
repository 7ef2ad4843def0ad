"""minikv_decode_attn_noalloc: the decode entry point that allocates nothing
(its split partials live in the library's per-device scratch array).  Its
results must equal minikv_decode_attn's with a caller workspace, on two calls
in a row, the second on a smaller cache (the array keeps the first call's
contents); and a call whose partials would not fit is rejected on the host.
The library's decode output is itself checked against the oracle in
test_gpu_decode.py; here it is the reference."""
import ctypes

import numpy as np
import pytest

from bit_quantized_attention_two_amd import synth
from gpu_util import dev16, require_gpu, say


def _cache(torch, mk, B, Hkv, g, D, n, m, seed, res):
    k, v = synth.gen_kv(seed, B * Hkv, n, D)
    sel = synth.gen_selection(seed, B * Hkv, n, m)
    dims = mk.make_dims(B, Hkv * g, Hkv, D)
    cache = mk.LayerCache(dims, (m // 16) * 16 + 256)
    kd = dev16(torch, k.reshape(B, Hkv, n, D))
    vd = dev16(torch, v.reshape(B, Hkv, n, D))
    mk.pack(dims, kd, vd, torch.from_numpy(sel.reshape(B, Hkv, m)).cuda(),
            cache)
    for t in range(res):
        mk.append(dims, cache, kd[:, :, t].contiguous(), vd[:, :, t].contiguous())
    return dims, cache


@pytest.mark.gpu
def test_noalloc_equals_workspace_decode_twice():
    torch, mk = require_gpu()
    cases = [dict(B=4, Hkv=8, g=4, D=128, n=3000, m=2100, seed=71, res=37),
             dict(B=1, Hkv=2, g=2, D=64, n=300, m=150, seed=72, res=3)]
    for case in cases:                 # the second call is the smaller one
        say("noalloc", case)
        dims, cache = _cache(torch, mk, **case)
        q, _, _ = synth.gen_decode_step(9, 0, case["seed"], case["B"],
                                        case["Hkv"] * case["g"], case["Hkv"],
                                        case["D"])
        qd = dev16(torch, q)
        ref = mk.decode_attn(dims, cache, qd)
        got = mk.decode_attn_noalloc(dims, cache, qd)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), case
        assert torch.isfinite(got.float()).all()


def test_noalloc_rejects_partials_beyond_scratch():
    """Host validation, no GPU needed: 4096 kv heads x g 8 x D 128 with 8192
    packed tokens would need far more than the 16 MiB array."""
    from bit_quantized_attention_two_amd import minikv as mk
    L = mk.lib()
    d = mk.make_dims(512, 8 * 8, 8, 128)
    fake = 0x1000
    c = mk._CacheC(*([fake] * 8), 8192, 8192, 0)
    P = ctypes.c_void_p
    rc = L.minikv_decode_attn_noalloc(ctypes.byref(d), ctypes.byref(c),
                                      P(fake), P(fake), None)
    assert rc == mk.ECAPACITY and b"scratch" in L.minikv_last_error()
    c2 = mk._CacheC(*([fake] * 8), 64, 0, 0)
    rc = L.minikv_decode_attn_noalloc(ctypes.byref(d), ctypes.byref(c2),
                                      P(fake), P(fake), None)
    assert rc == mk.EINVAL
