"""Write the oracle's per-key cumulative scores of whole full-size units.

    python tests/golden/make_golden_scores.py [config ...]

For each listed unit (workload, layer, batch element, kv head) this runs the
CPU oracle's plain row-by-row prefill (oracle.prefill_rows: fp64 softmax of
every causal query row of the kv head's g query heads, each row's
probabilities added into its columns) over ALL n query rows, on the seeded
synthetic inputs the GPU tests draw (synth.gen_unit_batch), and saves the
resulting score of every key as float64 .npy next to this script, with a
JSON note of what it holds.  Only oracle/ and the input generator are used.

Rows are split over threads by residue (row i goes to thread i mod T, which
balances the causal work); each thread adds into its own score vector and
the T vectors are summed in thread order, so the result does not depend on
scheduling.  The 131072-token unit takes ~15 minutes on 8 cores.
"""
import concurrent.futures as cf
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from bit_quantized_attention_two_amd import configs, synth  # noqa: E402

# (workload id, layer, batch element, kv head)
UNITS = {
    3: [(3, 0, 0, 0), (3, 0, 15, 39)],
    4: [(4, 0, 0, 0)],
    5: [(5, 0, 0, 0)],
}


# DiffKV's significance: per-head column sums, max over the group's heads
# (the significance is that maximum over n - j)
COLMAX_UNITS = {4: [(4, 0, 0, 0)]}


def golden_path(cfg_id, layer, b, h):
    name = configs.get(cfg_id)["name"].replace("-", "_")
    return os.path.join(HERE, "scores_%s_l%d_b%d_h%d.npy" % (name, layer, b, h))


def unit_inputs(cfg_id, layer, b, h):
    c = configs.get(cfg_id)
    r_window = c["n"] * c["rw"][0] // c["rw"][1]
    q, k, v = synth.gen_unit_batch(cfg_id, layer, b, c["Hq"], c["Hkv"], c["n"],
                                   c["D"], r_window)
    g = c["g"]
    return (np.ascontiguousarray(q[h * g:(h + 1) * g]),
            np.ascontiguousarray(k[h]), np.ascontiguousarray(v[h]))


def oracle_scores(q, k, v, threads):
    n = q.shape[1]
    parts = [np.arange(t, n, threads, dtype=np.int32) for t in range(threads)]
    with cf.ThreadPoolExecutor(threads) as ex:
        cols = list(ex.map(lambda rows: oracle.prefill_rows(
            q, k, v, rows, want_o=False, want_lse=False)[2], parts))
    total = np.zeros(n, np.float64)
    for col in cols:                    # fixed order
        total += col
    return total


def colmax_path(cfg_id, layer, b, h):
    name = configs.get(cfg_id)["name"].replace("-", "_")
    return os.path.join(HERE, "colmax_%s_l%d_b%d_h%d.npy" % (name, layer, b, h))


def write_colmax(cfg_id, threads):
    for cfg_id_, layer, b, h in COLMAX_UNITS.get(cfg_id, []):
        t0 = time.time()
        q, k, v = unit_inputs(cfg_id_, layer, b, h)
        cols = [oracle_scores(np.ascontiguousarray(q[i:i + 1]), k, v, threads)
                for i in range(q.shape[0])]
        colmax = np.max(np.stack(cols), axis=0)
        path = colmax_path(cfg_id_, layer, b, h)
        np.save(path, colmax)
        c = configs.get(cfg_id_)
        with open(path[:-4] + ".json", "w") as f:
            json.dump({
                "what": "oracle per-key column sum of each query head of the "
                        "unit's group, max over the g heads, fp64 (DiffKV's "
                        "significance times n - j)",
                "workload": c["name"], "layer": layer, "batch": b, "kv_head": h,
                "n": c["n"], "g": c["g"], "D": c["D"],
                "inputs": "bit_quantized_attention_two_amd.synth."
                          "gen_unit_batch(%d, %d, %d, ...)" % (cfg_id_, layer, b),
                "writer": "tests/golden/make_golden_scores.py (oracle only)",
            }, f, indent=1)
        print("%s: %.1f s" % (os.path.basename(path), time.time() - t0), flush=True)


def main(ids, colmax_only=False):
    oracle.build(force=False)
    threads = os.cpu_count() or 1
    for cfg_id in ids:
        write_colmax(cfg_id, threads)
    if colmax_only:
        return
    for cfg_id in ids:
        for cfg_id_, layer, b, h in UNITS[cfg_id]:
            t0 = time.time()
            q, k, v = unit_inputs(cfg_id_, layer, b, h)
            col = oracle_scores(q, k, v, threads)
            path = golden_path(cfg_id_, layer, b, h)
            np.save(path, col)
            c = configs.get(cfg_id_)
            note = {
                "what": "oracle per-key cumulative attention score of one "
                        "unit: col[j] = sum over the kv head's g query heads "
                        "and all causal rows i >= j of softmax(q_i k^T / "
                        "sqrt(D))[j], fp64",
                "workload": c["name"], "layer": layer, "batch": b,
                "kv_head": h, "n": c["n"], "g": c["g"], "D": c["D"],
                "inputs": "bit_quantized_attention_two_amd.synth."
                          "gen_unit_batch(%d, %d, %d, ...)" % (cfg_id_, layer, b),
                "writer": "tests/golden/make_golden_scores.py (oracle only)",
                "sum": float(col.sum()),
            }
            with open(path[:-4] + ".json", "w") as f:
                json.dump(note, f, indent=1)
            print("%s: sum %.9f (g n = %d), %.1f s" % (
                os.path.basename(path), col.sum(), c["g"] * c["n"],
                time.time() - t0), flush=True)


if __name__ == "__main__":
    args = [a for a in sys.argv[1:] if a != "--colmax-only"]
    main([int(x) for x in args] or sorted(UNITS), "--colmax-only" in sys.argv)
