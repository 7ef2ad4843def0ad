"""The fused prefill tail (minikv_prefill_select_pack: the selection inside
the second prefill pass, or after it, then the pack) against the separate calls
(minikv_prefill_select, then minikv_pack), bit for bit: attention output,
cumulative scores, selection and every packed array; the separate calls are
themselves checked against the oracle in the other GPU tests.  Shapes from
one unit to many (the XCD-ordered grids), every workload's layer-0 shape at
reduced batch, and the empty-selection edge cases."""
import numpy as np
import pytest

from bit_quantized_attention_two_amd import synth
from gpu_util import cache_to_numpy, dev16, require_gpu, say

pytestmark = pytest.mark.gpu


def _run_both(torch, mk, q, k, v, n_hh, n_recent, Gk=16):
    B, Hq, n, D = q.shape
    Hkv = k.shape[1]
    dims = mk.make_dims(B, Hq, Hkv, D, Gk)
    qd, kd, vd = dev16(torch, q), dev16(torch, k), dev16(torch, v)
    m = n_hh + n_recent
    cap = (m // Gk) * Gk + Gk
    c1, c2 = mk.LayerCache(dims, cap), mk.LayerCache(dims, cap)
    o1, col1, sel1 = mk.prefill_select(dims, qd, kd, vd, n_hh, n_recent)
    mk.pack(dims, kd, vd, sel1, c1)
    # a dirty workspace: the counters must not depend on its contents
    ws = torch.full((mk.prefill_tail_ws_bytes(dims, n),), 0x5a, dtype=torch.uint8,
                    device="cuda")
    for rep in range(3):                   # the counters reset between calls
        fuse = rep < 2
        o2, col2, sel2 = mk.prefill_select_pack(dims, qd, kd, vd, n_hh, n_recent, c2,
                                                fuse_select=fuse, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(col1, col2), rep
        assert torch.equal(sel1, sel2), rep
        a, b = cache_to_numpy(c1), cache_to_numpy(c2)
        assert (c1.n_packed, c1.n_res) == (c2.n_packed, c2.n_res)
        for name in a:
            assert np.array_equal(a[name], b[name]), (rep, name)


@pytest.mark.parametrize("B,Hq,Hkv,D,n,hh,rw", [
    (1, 1, 1, 64, 1, 0, 1), (1, 2, 2, 128, 37, 9, 9), (2, 4, 2, 64, 300, 75, 75),
    (1, 4, 4, 64, 256, 64, 64), (2, 8, 8, 128, 4096, 1902, 1024),
    (8, 8, 8, 128, 1000, 250, 250), (1, 8, 2, 128, 6000, 1500, 1500),
    (1, 4, 1, 128, 513, 0, 128), (1, 4, 1, 128, 513, 385, 0),
])
def test_fused_tail_equals_separate_calls(B, Hq, Hkv, D, n, hh, rw):
    torch, mk = require_gpu()
    say("fused-tail", dict(B=B, Hq=Hq, Hkv=Hkv, D=D, n=n, hh=hh, rw=rw))
    q, k, v = [], [], []
    for b in range(B):
        a = synth.gen_unit_batch(2, 5, b, Hq, Hkv, n, D, rw)
        q.append(a[0]); k.append(a[1]); v.append(a[2])
    _run_both(torch, mk, np.stack(q), np.stack(k), np.stack(v), hh, rw)


def test_fused_tail_capacity_error_has_no_side_effect():
    torch, mk = require_gpu()
    dims = mk.make_dims(1, 2, 2, 128)
    q = torch.zeros((1, 2, 300, 128), dtype=torch.float16, device="cuda")
    cache = mk.LayerCache(dims, 64)
    with pytest.raises(mk.MiniKVError) as e:
        mk.prefill_select_pack(dims, q, q, q, 75, 75, cache, fuse_select=True)
    assert e.value.status == mk.ECAPACITY and cache.n_packed == 0
