"""Writes the hand-derived fixtures in this folder.

Every expected value below is a closed form worked out by hand (the pages
print no numeric worked example); the script only formats them as JSON.  It
calls neither the oracle nor the HIP library.  Run: python tests/golden/make_golden.py
"""
import json
import math
import os

ln = math.log
HERE = os.path.dirname(os.path.abspath(__file__))


def write(name, obj):
    with open(os.path.join(HERE, name), "w") as f:
        json.dump(obj, f, indent=1)
        f.write("\n")


write("softmax_hand.json", {
    "source": "Hand-derived closed form (no worked example is printed on the pages). "
              "Definition followed: one softmax over all visible keys per query row "
              "[Ring Attention Q&A, aivaro.ru answer 425, sections 1-2]; causal visibility "
              "key_pos <= query_pos. Scores are chosen as logs of small integers so the "
              "softmax weights are exact rationals.",
    "scale": 1.0,
    "q": [[[[1.0, 0.0], [0.0, 1.0]]]],
    "k": [[[[0.0, ln(4)], [ln(2), 0.0], [ln(3), 0.0]]]],
    "v": [[[[6.0, 0.0], [0.0, 6.0], [6.0, 6.0]]]],
    "noncausal": {
        "derivation": "row0 scores (0, ln2, ln3) -> weights (1,2,3)/6 -> O=(6*1+0*2+6*3, 0*1+6*2+6*3)/6=(4,5), lse=ln6; "
                      "row1 scores (ln4, 0, 0) -> weights (4,1,1)/6 -> O=(24+0+6, 0+6+6)/6=(5,2), lse=ln6",
        "O": [[[[4.0, 5.0], [5.0, 2.0]]]],
        "lse": [[[ln(6), ln(6)]]],
    },
    "causal_q0_k0": {
        "derivation": "q_pos0=k_pos0=0: row0 sees key0 only -> O=v0=(6,0), lse=s00=0; "
                      "row1 sees keys 0,1 with scores (ln4, 0) -> weights (4,1)/5 -> O=(24/5, 6/5), lse=ln5",
        "O": [[[[6.0, 0.0], [4.8, 1.2]]]],
        "lse": [[[0.0, ln(5)]]],
    },
    "causal_q_behind_keys": {
        "derivation": "q_pos0=0, k_pos0=1: row0 sees no key -> O=0, lse=-inf; row1 sees key0 only -> O=v0=(6,0), lse=s10=ln4",
        "O": [[[[0.0, 0.0], [6.0, 0.0]]]],
        "lse": [[["-inf", ln(4)]]],
    },
})

write("ulysses_hand.json", {
    "source": "Hand-derived from the Ulysses all_to_all description [Ulysses post, stuffynlp 213]: "
              "shard p holds tokens p*n..p*n+n-1 for all heads; rank r receives heads r*H/P.. for the "
              "whole sequence, pieces concatenated in source-rank order; GQA KV heads are copied "
              "(repeat-interleave) up to the group size. Element value = 10*token + head.",
    "P": 2, "L": 4, "d": 1,
    "cases": [
        {"H_src": 2, "H_dst": 2,
         "src": [[[[0], [1]], [[10], [11]]], [[[20], [21]], [[30], [31]]]],
         "dst": [[[[0]], [[10]], [[20]], [[30]]], [[[1]], [[11]], [[21]], [[31]]]]},
        {"H_src": 1, "H_dst": 2,
         "src": [[[[0]], [[10]]], [[[20]], [[30]]]],
         "dst": [[[[0]], [[10]], [[20]], [[30]]], [[[0]], [[10]], [[20]], [[30]]]]},
        {"H_src": 2, "H_dst": 4,
         "src": [[[[0], [1]], [[10], [11]]], [[[20], [21]], [[30], [31]]]],
         "dst": [[[[0], [0]], [[10], [10]], [[20], [20]], [[30], [30]]],
                 [[[1], [1]], [[11], [11]], [[21], [21]], [[31], [31]]]]},
    ],
})

write("attn_matrix_memory.json", {
    "source": "accelerate concept guide 'Paralelismo de secuencias en 🤗 accelerate', section "
              "'¿Por qué la paralelización de secuencias?': at a 128k sequence a standard bf16 attention "
              "materialises 128k*128k*2 bytes per head, printed as about 32 GB per head.",
    "L": 131072, "elem_bytes": 2, "heads": 1,
    "printed_GB_per_head": 32,
    "exact_bytes_per_head": 131072 * 131072 * 2,
})
