"""Pins of the oracle's prefill (attention output, LSE, cumulative scores).

- torch's scaled_dot_product_attention (causal, fp64, CPU) -- a library
  implementation -- for the output on tiny inputs;
- torch.logsumexp / torch.softmax of the causally masked logit matrix for LSE
  and the per-key column sums on tiny inputs (brute force n x n);
- the closed form for K == 0 (uniform causal attention): o_i is the running
  mean of v, LSE_i = ln(i+1), col_j = g * (H_n - H_j) with harmonic numbers;
- the invariant sum_j col_j = g * n (every softmax row sums to one);
- the edges o_0 = v_0, LSE_0 = q_0.k_0 / sqrt(D).
"""
import numpy as np
import pytest
import torch

from bit_quantized_attention_two_amd import synth


def _torch_ref(q, k, v):
    q64 = torch.from_numpy(q.astype(np.float64))
    k64 = torch.from_numpy(k.astype(np.float64))
    v64 = torch.from_numpy(v.astype(np.float64))
    g, n, D = q64.shape
    o = torch.nn.functional.scaled_dot_product_attention(
        q64, k64.expand(g, n, D), v64.expand(g, n, D), is_causal=True)
    s = (q64 @ k64.T) / np.sqrt(D)
    mask = torch.ones(n, n, dtype=torch.bool).tril()
    s = s.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    col = torch.softmax(s, dim=-1).sum(dim=(0, 1))
    return o.numpy(), lse.numpy(), col.numpy()


@pytest.mark.parametrize("n,D,g", [(1, 16, 1), (7, 16, 2), (33, 64, 1),
                                   (64, 64, 4), (100, 16, 3)])
def test_prefill_vs_torch_bruteforce(oracle, n, D, g):
    r = np.random.default_rng(n * 1000 + D + g)
    q = (r.standard_normal((g, n, D)) * 1.5).astype(np.float16)
    k = (r.standard_normal((n, D)) * 1.5).astype(np.float16)
    v = r.standard_normal((n, D)).astype(np.float16)
    o, lse, col = oracle.prefill_unit(q, k, v)
    ro, rl, rc = _torch_ref(q, k, v)
    np.testing.assert_allclose(o, ro, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(col, rc, rtol=1e-11, atol=1e-12)


def test_prefill_structured_synthetic_vs_torch(oracle):
    q, k, v = synth.gen_unit_batch(1, 0, 0, Hq=4, Hkv=2, n=96, D=64,
                                   r_window=24)
    for h in range(2):
        o, lse, col = oracle.prefill_unit(q[2 * h:2 * h + 2], k[h], v[h])
        ro, rl, rc = _torch_ref(q[2 * h:2 * h + 2], k[h], v[h])
        np.testing.assert_allclose(o, ro, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(lse, rl, rtol=1e-12)
        np.testing.assert_allclose(col, rc, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("g", [1, 4])
def test_prefill_zero_keys_closed_form(oracle, g):
    n, D = 50, 16
    r = np.random.default_rng(1)
    q = r.standard_normal((g, n, D)).astype(np.float16)
    k = np.zeros((n, D), np.float16)
    v = r.standard_normal((n, D)).astype(np.float16)
    o, lse, col = oracle.prefill_unit(q, k, v)
    vd = v.astype(np.float64)
    run_mean = np.cumsum(vd, axis=0) / np.arange(1, n + 1)[:, None]
    for h in range(g):
        np.testing.assert_allclose(o[h], run_mean, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse[h], np.log(np.arange(1, n + 1)),
                                   rtol=1e-14, atol=1e-15)
    H = np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, n + 1))])
    np.testing.assert_allclose(col, g * (H[n] - H[:n]), rtol=1e-13)


def test_prefill_col_sums_to_gn_and_edges(oracle):
    n, D, g = 80, 64, 2
    r = np.random.default_rng(9)
    q = (r.standard_normal((g, n, D)) * 3).astype(np.float16)
    k = (r.standard_normal((n, D)) * 3).astype(np.float16)
    v = r.standard_normal((n, D)).astype(np.float16)
    o, lse, col = oracle.prefill_unit(q, k, v)
    assert abs(col.sum() - g * n) < 1e-9 * g * n
    np.testing.assert_array_equal(o[:, 0], np.broadcast_to(
        v[0].astype(np.float64), (g, D)))
    qd, kd = q.astype(np.float64), k.astype(np.float64)
    np.testing.assert_allclose(lse[:, 0], qd[:, 0] @ kd[0] / np.sqrt(D),
                               rtol=1e-14)
    # col[n-1] is the diagonal probability of the last row, summed over heads
    last = 0.0
    for h in range(g):
        s = qd[h, n - 1] @ kd.T / np.sqrt(D)
        p = np.exp(s - s.max())
        last += p[-1] / p.sum()
    assert abs(col[n - 1] - last) < 1e-13


def test_prefill_row_subset_matches_full(oracle):
    n, D, g = 64, 16, 2
    r = np.random.default_rng(2)
    q = r.standard_normal((g, n, D)).astype(np.float16)
    k = r.standard_normal((n, D)).astype(np.float16)
    v = r.standard_normal((n, D)).astype(np.float16)
    o, lse, col = oracle.prefill_unit(q, k, v)
    rows = np.array([63, 0, 17, 40], np.int32)
    o2, l2, c2 = oracle.prefill_rows(q, k, v, rows)
    np.testing.assert_array_equal(o2, o[:, rows])
    np.testing.assert_array_equal(l2, lse[:, rows])
    # the last rows alone give the tail columns exactly
    tail = np.arange(48, 64, dtype=np.int32)
    _, _, c3 = oracle.prefill_rows(q, k, v, tail, want_o=False, want_lse=False)
    np.testing.assert_allclose(c3[48:], col[48:], rtol=1e-14)
