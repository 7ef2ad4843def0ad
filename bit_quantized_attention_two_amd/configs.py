"""The five synthetic workloads the library is tested and measured on.

Shapes follow the models and context lengths of the MiniKV pages' runs
(Pith review of MiniKV, "The reading" and referee major comments: LLaMA2-7B/13B,
Mistral-7B, Llama-3, LongBench truncated to 4096 tokens, InfiniteBench long
contexts).  Budgets follow "Assumptions & free parameters" on the same page:
25% heavy hitters + 25% recent window of the prompt per layer, pyramid depth 7,
group size 16, residual buffer 128.
"""

SEED = 241118077          # the MiniKV arXiv id, as the base of every seed tuple

COMMON = dict(depth=7, hh=(1, 4), rw=(1, 4), residual_cap=128)

CONFIGS = {
    1: dict(name="tiny-1layer", B=1, Hq=4, Hkv=4, D=64, n=256, L=1,
            pyramid=False, Gk=32, Gv=16, decode_steps=16),
    2: dict(name="llama2-7b-4k", B=1, Hq=32, Hkv=32, D=128, n=4096, L=32,
            pyramid=True, Gk=16, Gv=16, decode_steps=128),
    3: dict(name="llama2-13b-b16-8k", B=16, Hq=40, Hkv=40, D=128, n=8192,
            L=40, pyramid=False, Gk=16, Gv=16, decode_steps=256),
    4: dict(name="mistral-7b-gqa-b4-32k", B=4, Hq=32, Hkv=8, D=128, n=32768,
            L=32, pyramid=True, Gk=16, Gv=16, decode_steps=128),
    5: dict(name="llama3-8b-gqa-128k", B=1, Hq=32, Hkv=8, D=128, n=131072,
            L=32, pyramid=True, Gk=16, Gv=16, decode_steps=64),
}


def get(cfg_id):
    c = dict(COMMON)
    c.update(CONFIGS[cfg_id])
    c["id"] = cfg_id
    c["g"] = c["Hq"] // c["Hkv"]
    return c
