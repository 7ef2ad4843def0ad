"""Helpers shared by the GPU parity tests (not collected by pytest)."""
import sys

import numpy as np
import pytest

ATOL, RTOL = 2e-3, 1e-3     # |gpu - ref| <= ATOL + RTOL * |ref|


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bit_quantized_attention_two_amd import minikv
    minikv.lib()                 # fails loudly if the HIP library is missing
    return torch, minikv


def say(*a):
    """Name the case on stdout before each GPU step (flushed)."""
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def dev16(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.float16)).cuda()


def assert_close(gpu, ref, what, atol=ATOL, rtol=RTOL):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), "%s: non-finite GPU values" % what
    err = np.abs(gpu - ref)
    bound = atol + rtol * np.abs(ref)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError("%s: %d/%d outside tolerance; worst at %s gpu=%r "
                             "ref=%r" % (what, int(bad.sum()), bad.size, i,
                                         gpu[i], ref[i]))
    return float((err / bound).max()) if err.size else 0.0


def cache_to_numpy(cache):
    """Packed arrays of a minikv.LayerCache as numpy (uint32/uint16 views)."""
    out = {}
    for name in cache.NAMES:
        t = getattr(cache, name).cpu().numpy()
        out[name] = t.view(np.uint32) if t.dtype == np.int32 else t.view(np.uint16)
    return out


ORACLE_NAMES = {"kq": "kq", "k_scale": "ks", "k_zero": "kz", "vq": "vq",
                "v_scale": "vs", "v_zero": "vz", "k_res": "kres",
                "v_res": "vres"}


def assert_cache_equal(gpu_cache, ocache, B, Hkv):
    """Bit-exact comparison of the valid parts of a GPU cache and an
    OracleCache of the same shape."""
    assert gpu_cache.n_packed == ocache.n_packed
    assert gpu_cache.n_res == ocache.n_res
    g = cache_to_numpy(gpu_cache)
    npk, nres = ocache.n_packed, ocache.n_res
    Gk = ocache.Gk
    sl = {"kq": np.s_[:, :, :npk], "k_scale": np.s_[:, :, :npk // Gk],
          "k_zero": np.s_[:, :, :npk // Gk], "vq": np.s_[:, :, :npk // 16],
          "v_scale": np.s_[:, :, :npk], "v_zero": np.s_[:, :, :npk],
          "k_res": np.s_[:, :, :nres], "v_res": np.s_[:, :, :nres]}
    for name, oname in ORACLE_NAMES.items():
        ga = g[name].reshape((B, Hkv) + g[name].shape[1:])[sl[name]]
        oa = getattr(ocache, oname)[sl[name]]
        if not np.array_equal(ga, oa):
            idx = np.argwhere(ga != oa)
            raise AssertionError("%s differs at %d places, first %s gpu=%r "
                                 "oracle=%r" % (name, len(idx), idx[0],
                                                ga[tuple(idx[0])],
                                                oa[tuple(idx[0])]))


def lib_budgets(mk, c, n=None, n_layers=None):
    """The library's per-layer budgets (minikv_pyramid_budgets) for workload
    c, asserted equal to the oracle's before use."""
    import oracle
    n = c["n"] if n is None else n
    L = c["L"] if n_layers is None else n_layers
    ks, r = mk.pyramid_budgets(n, L, c["hh"], c["rw"], c["depth"], c["pyramid"])
    oks, orr = oracle.budgets(n, L, c["depth"], c["pyramid"], c["hh"], c["rw"])
    assert r == orr and list(ks) == list(oks), "library budgets differ from the oracle's"
    return np.asarray(ks, np.int32), r
