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


def topk_of(col, n_hh, n_recent):
    n = col.size
    cand = np.arange(n - n_recent)
    order = np.lexsort((cand, -col[:n - n_recent].astype(np.float64)))
    return np.concatenate([np.sort(cand[order[:n_hh]]),
                           np.arange(n - n_recent, n)]).astype(np.int32)


def check_selection(gsel, gcol, osel, ocol, n_hh, n_recent):
    """Selection protocol.  (1) The oracle's selection applied to the GPU's
    own scores must be the GPU's selection exactly (the set is unique given
    the scores, ties to the lower index).  (2) Against the oracle's
    selection on its own scores, a difference is accepted only as swaps of
    boundary candidates whose oracle scores agree with the k-th score within
    the score tolerance.  Returns the number of swaps."""
    import oracle
    assert np.array_equal(gsel, oracle.select(np.asarray(gcol, np.float64),
                                              n_hh, n_recent))
    assert np.array_equal(gsel, topk_of(gcol, n_hh, n_recent))
    if osel is None:
        return 0
    # (2) against the oracle's selection: only boundary swaps
    if np.array_equal(gsel, osel):
        return 0
    a, b = set(gsel.tolist()), set(osel.tolist())
    only_g, only_o = sorted(a - b), sorted(b - a)
    assert len(only_g) == len(only_o)
    kth = np.sort(ocol[:ocol.size - n_recent])[::-1][n_hh - 1]
    for j in only_g + only_o:
        assert abs(ocol[j] - kth) <= ATOL + RTOL * abs(kth), (j, ocol[j], kth)
    return len(only_g)
