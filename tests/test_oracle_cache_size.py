"""Pin of the closed-form cache size against the numbers the MiniKV pages
print (tests/golden/cache_size_llama2_7b.json, with its citation)."""
import json
import math
import os

GOLDEN = os.path.join(os.path.dirname(__file__), "golden",
                      "cache_size_llama2_7b.json")


def test_cache_size_matches_printed_numbers(oracle):
    g = json.load(open(GOLDEN))
    s = g["model_shape"]
    mini, full = oracle.cache_bytes(s["n_layers"], s["n_heads"], s["head_dim"],
                                    g["lprompt"], g["lgen"], g["budget_frac"],
                                    g["bits"], g["group"])
    p = g["printed"]
    # the page prints the sizes cut to its digits (0.3355 GB -> "0.33")
    assert math.floor(mini / 1e9 * 100) / 100 == p["minikv_gb"]
    assert math.floor(full / 1e9 * 10) / 10 == p["full_gb"]
    assert round(100 * (1 - mini / full)) == p["reduction_pct"]
    # exact byte counts of the reading (both K and V at 4 bits/element)
    assert mini == 335544320 and full == 2415919104


def test_cache_size_codes_only_would_not_match(oracle):
    """Dropping the fp16 scale/zero term (a plausible slip) misses the
    printed 0.33 GB, so the golden numbers do constrain the formula."""
    g = json.load(open(GOLDEN))
    s = g["model_shape"]
    mini, _ = oracle.cache_bytes(s["n_layers"], s["n_heads"], s["head_dim"],
                                 g["lprompt"], g["lgen"], g["budget_frac"],
                                 g["bits"], 10 ** 9)
    assert math.floor(mini / 1e9 * 100) / 100 != g["printed"]["minikv_gb"]
