"""GPU parity of minikv_prefill_attn (O, LSE, per-key cumulative scores) and
minikv_select against the oracle.

O, LSE and col: |gpu - ref| <= 2e-3 + 1e-3 |ref| against the fp64 oracle;
sum_j col_j = g n on every unit (rows of a softmax sum to one).  Selection on
seeded score vectors: bit-exact indices."""
import concurrent.futures as cf
import os

import numpy as np
import pytest

import oracle
from bit_quantized_attention_two_amd import synth
from gpu_util import assert_close, dev16, require_gpu, say

pytestmark = pytest.mark.gpu

WORKERS = min(16, os.cpu_count() or 1)


def _prefill(torch, mk, q, k, v, Gk=16):
    B, Hq, n, D = q.shape
    Hkv = k.shape[1]
    dims = mk.make_dims(B, Hq, Hkv, D, Gk)
    o, lse, col = mk.prefill_attn(dims, dev16(torch, q), dev16(torch, k),
                                  dev16(torch, v))
    return (o.cpu().numpy().astype(np.float64), lse.cpu().numpy(),
            col.cpu().numpy())


def _oracle_units(q, k, v, units, rows=None):
    B, Hq, n, D = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv

    def one(u):
        b, h = u
        rr = np.arange(n, dtype=np.int32) if rows is None else rows
        return oracle.prefill_rows(q[b, h * g:(h + 1) * g], k[b, h], v[b, h], rr)

    with cf.ThreadPoolExecutor(WORKERS) as ex:
        return list(ex.map(one, units))


@pytest.mark.parametrize("B,Hq,Hkv,D,n", [
    (1, 1, 1, 64, 1), (1, 2, 2, 128, 37), (2, 4, 2, 64, 128),
    (1, 4, 1, 128, 200), (2, 8, 1, 128, 300), (1, 8, 4, 64, 513),
    (1, 4, 4, 64, 256),                      # tiny single-layer workload shape
])
def test_prefill_small_all_units(B, Hq, Hkv, D, n):
    torch, mk = require_gpu()
    q, k, v = [], [], []
    for b in range(B):
        a = synth.gen_unit_batch(1, 0, b, Hq, Hkv, n, D, n // 4)
        q.append(a[0]); k.append(a[1]); v.append(a[2])
    q, k, v = np.stack(q), np.stack(k), np.stack(v)
    say("prefill-small", dict(B=B, Hq=Hq, Hkv=Hkv, D=D, n=n))
    o, lse, col = _prefill(torch, mk, q, k, v)
    g = Hq // Hkv
    units = [(b, h) for b in range(B) for h in range(Hkv)]
    for (b, h), (ro, rl, rc) in zip(units, _oracle_units(q, k, v, units)):
        assert_close(o[b, h * g:(h + 1) * g], ro, "O b%d h%d" % (b, h))
        assert_close(lse[b, h * g:(h + 1) * g], rl, "LSE b%d h%d" % (b, h))
        assert_close(col[b, h], rc, "col b%d h%d" % (b, h))
    np.testing.assert_allclose(col.sum(-1), g * n, rtol=1e-4)


@pytest.mark.parametrize("B,Hq,Hkv,n", [(8, 32, 32, 1000), (16, 8, 4, 4000)])
def test_prefill_many_units(B, Hq, Hkv, n):
    """Enough units and keys that pass 2 takes its 64-keys-per-wave form;
    four units (first, last, two inner) are compared on every row and
    column, and every unit must satisfy sum(col) = g n."""
    torch, mk = require_gpu()
    D = 128
    assert B * Hkv * ((n + 255) // 256) >= 1024
    q, k, v = [], [], []
    for b in range(B):
        a = synth.gen_unit_batch(2, 0, b, Hq, Hkv, n, D, n // 4)
        q.append(a[0]); k.append(a[1]); v.append(a[2])
    q, k, v = np.stack(q), np.stack(k), np.stack(v)
    say("prefill-many", dict(B=B, Hq=Hq, Hkv=Hkv, D=D, n=n))
    o, lse, col = _prefill(torch, mk, q, k, v)
    g = Hq // Hkv
    np.testing.assert_allclose(col.sum(-1), g * n, rtol=1e-4)
    units = [(0, 0), (B - 1, Hkv - 1), (B // 2, 1), (1, Hkv // 2)]
    for (b, h), (ro, rl, rc) in zip(units, _oracle_units(q, k, v, units)):
        assert_close(o[b, h * g:(h + 1) * g], ro, "O b%d h%d" % (b, h))
        assert_close(lse[b, h * g:(h + 1) * g], rl, "LSE b%d h%d" % (b, h))
        assert_close(col[b, h], rc, "col b%d h%d" % (b, h))


@pytest.mark.parametrize("cfg_id,full_units,rows", [(2, 2, 48), (4, 1, 24),
                                                    (5, 1, 12)])
def test_prefill_full_size(cfg_id, full_units, rows):
    """One layer at the workload's real size (batch element 0): the oracle
    evaluates `rows` random query rows plus the last 64 rows (which fix the
    last 64 columns of col exactly) on `full_units` units, and every unit
    must satisfy sum(col) = g n."""
    torch, mk = require_gpu()
    from bit_quantized_attention_two_amd import configs
    c = configs.get(cfg_id)
    q, k, v = synth.gen_prefill(cfg_id, 0, batches=[0])
    n, g = c["n"], c["g"]
    say("prefill-full", dict(cfg=cfg_id, n=n, Hq=c["Hq"], Hkv=c["Hkv"]))
    o, lse, col = _prefill(torch, mk, q, k, v)
    np.testing.assert_allclose(col.sum(-1), g * n, rtol=1e-4)
    rr = np.random.default_rng(cfg_id)
    sample = np.unique(np.concatenate([rr.choice(n - 64, rows, replace=False),
                                       np.arange(n - 64, n)])).astype(np.int32)
    units = [(0, h) for h in rr.choice(c["Hkv"], full_units, replace=False)]
    for (b, h), (ro, rl, rc) in zip(units, _oracle_units(q, k, v, units,
                                                         sample)):
        assert_close(o[b, h * g:(h + 1) * g][:, sample], ro, "O h%d" % h)
        assert_close(lse[b, h * g:(h + 1) * g][:, sample], rl, "LSE h%d" % h)
        assert_close(col[b, h, n - 64:], rc[n - 64:], "col tail h%d" % h)


# --------------------------------------------------------------- selection --

@pytest.mark.parametrize("kind", ["random", "ties", "const", "decreasing"])
@pytest.mark.parametrize("n,n_hh,n_recent", [
    (1, 0, 1), (1, 1, 0), (37, 9, 9), (256, 64, 64), (300, 0, 75),
    (300, 225, 75), (4096, 1902, 1024), (4096, 146, 1024),
    (32768, 15214, 8192), (131072, 60855, 32768), (5000, 4999, 0),
])
def test_select_bit_exact(kind, n, n_hh, n_recent):
    torch, mk = require_gpu()
    B, Hkv = 1, 3
    col = synth.gen_scores(n + n_hh, B * Hkv, n, kind)
    dims = mk.make_dims(B, Hkv, Hkv, 128)
    say("select", dict(kind=kind, n=n, n_hh=n_hh, n_recent=n_recent))
    sel = mk.select(dims, torch.from_numpy(col.reshape(B, Hkv, n)).cuda(),
                    n_hh, n_recent).cpu().numpy().reshape(B * Hkv, -1)
    for u in range(B * Hkv):
        ref = oracle.select(col[u].astype(np.float64), n_hh, n_recent)
        assert np.array_equal(sel[u], ref), (u, np.nonzero(sel[u] != ref)[0][:5])


def test_select_negative_and_signed_zero_scores():
    torch, mk = require_gpu()
    r = np.random.default_rng(4)
    col = r.standard_normal((2, 1000)).astype(np.float32)
    col[:, ::7] = 0.0
    col[:, 3::7] = -0.0
    dims = mk.make_dims(1, 2, 2, 128)
    sel = mk.select(dims, torch.from_numpy(col.reshape(1, 2, 1000)).cuda(),
                    400, 100).cpu().numpy().reshape(2, -1)
    for u in range(2):
        assert np.array_equal(sel[u], oracle.select(col[u].astype(np.float64),
                                                    400, 100))


def test_select_argument_errors():
    torch, mk = require_gpu()
    dims = mk.make_dims(1, 2, 2, 128)
    col = torch.zeros((1, 2, 10), dtype=torch.float32, device="cuda")
    with pytest.raises(mk.MiniKVError):
        mk.select(dims, col, 8, 3)
    with pytest.raises(mk.MiniKVError):
        mk.select(dims, col, 0, 11)
