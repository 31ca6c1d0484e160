"""Write the exact-arithmetic fixtures of tests/golden/.

Calls only the oracle package's brute force (oracle/bruteforce.py: rational
dot products, 60-digit decimal exponentials) on tiny seeded inputs from the
workload generators.  Run from the repository root:

    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle.bruteforce import attention_exact  # noqa: E402
from paged_gqa_kv_decode_amd.workloads import make_custom  # noqa: E402

CASES = {
    # name: (seq_lens, Hq, Hkv, D, bs, seed, sigma_k)
    "bf_gqa4_bs4.json": ([5, 9, 1], 8, 2, 8, 4, 901, 1.0),
    "bf_gqa6_peaky.json": ([7, 3], 6, 1, 4, 2, 902, 3.0),
    "bf_gqa8_ragged.json": ([11, 2, 8], 16, 2, 4, 8, 903, 1.0),
}


def main():
    here = os.path.dirname(os.path.abspath(__file__))
    for name, (lens, Hq, Hkv, D, bs, seed, sk) in CASES.items():
        wl = make_custom(seq_lens=lens, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                         block_size=bs, seed=seed, pool_factor=2.0, sigma_k=sk,
                         canaries=True)
        exact = attention_exact(wl.q, wl.k_cache, wl.v_cache, wl.block_tables,
                                wl.seq_lens, wl.scale)
        flat = [str(x) for s in exact for h in s for x in h]
        case = {
            "about": "exact softmax attention over paged fp16 K/V (oracle/bruteforce.py)",
            "shapes": {"q": list(wl.q.shape), "kv": list(wl.k_cache.shape)},
            "q_bits": wl.q.view(np.uint16).reshape(-1).tolist(),
            "k_bits": wl.k_cache.view(np.uint16).reshape(-1).tolist(),
            "v_bits": wl.v_cache.view(np.uint16).reshape(-1).tolist(),
            "block_tables": wl.block_tables.tolist(),
            "seq_lens": wl.seq_lens.tolist(),
            "scale": wl.scale,
            "expected": flat,
        }
        with open(os.path.join(here, name), "w") as f:
            json.dump(case, f)
        print("wrote", name, len(flat), "values")


if __name__ == "__main__":
    main()
