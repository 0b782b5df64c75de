"""Writes the hand-derived golden fixtures in this folder.

Every value here is a closed form worked by hand (stated in each file's
"source" field); nothing is computed by the oracle or the HIP path.
Run: python tests/golden/make_golden.py
"""
import json
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def main():
    g = {
        "source": "Hand-derived closed form. With Q = 0 every open key scores 0, so under a "
                  "causal mask row i averages V over keys 0..i and its logsumexp is ln(i+1). "
                  "Mask semantics: key j hides rows [0, j) (upper interval), the causal encoding "
                  "of the column-sparse form described on the FlashMask-3 page (predecessor paragraph).",
        "scale": 0.125,
        "k": [[0.5, -1.0], [2.0, 0.25], [-3.0, 1.5], [0.0, 4.0]],
        "v": [[1.0, 0.0], [3.0, 2.0], [5.0, -4.0], [7.0, 6.0]],
        "o": [[1.0, 0.0], [2.0, 1.0], [3.0, -2.0 / 3.0], [4.0, 1.0]],
        "lse": [0.0, math.log(2), math.log(3), math.log(4)],
    }
    w = {
        "source": "Hand-derived. d = 1, scale 1, every query is 1 and key j is ln(j+1), so the "
                  "score of (i, j) is ln(j+1) and exp(score) = j+1. Sliding window 2 (row i sees "
                  "keys i-1 and i): row 0 -> v0, lse 0; row 1 -> (1*v0 + 2*v1)/3, lse ln 3; "
                  "row 2 -> (2*v1 + 3*v2)/5, lse ln 5; row 3 -> (3*v2 + 4*v3)/7, lse ln 7.",
        "scale": 1.0, "window": 2,
        "q": [[1.0], [1.0], [1.0], [1.0]],
        "k": [[0.0], [math.log(2)], [math.log(3)], [math.log(4)]],
        "v": [[3.0], [6.0], [-4.0], [7.0]],
        "o": [[3.0], [5.0], [0.0], [16.0 / 7.0]],
        "lse": [0.0, math.log(3), math.log(5), math.log(7)],
    }
    loc = {
        "source": "Hand-worked localization: a global bound x becomes the number of the rank's "
                  "rows (ascending global order) whose global index is below x. This is the "
                  "result the clip/shift/max localization on the bound vectors must give "
                  "(FlashMask-3 page, contributions paragraph and 'Key facts').",
        "cases": [
            {"note": "rows {2,3,4,10,11,12,13} of 16", "seq_q_global": 16,
             "chunk_start": [2, 10], "chunk_len": [3, 4],
             "global": [-5, 0, 2, 3, 5, 7, 10, 11, 14, 16, 99],
             "local": [0, 0, 0, 1, 3, 3, 3, 4, 7, 7, 7]},
            {"note": "dual-chunk rank 3 of 8 over 65536 (chunks 3 and 12 of 4096)",
             "seq_q_global": 65536, "chunk_start": [12288, 49152], "chunk_len": [4096, 4096],
             "global": [0, 12288, 12289, 16384, 30000, 49152, 50000, 53248, 65536],
             "local": [0, 0, 1, 4096, 4096, 4096, 4944, 8192, 8192]},
            {"note": "one chunk covering everything is the identity inside [0, Sq]",
             "seq_q_global": 8, "chunk_start": [0], "chunk_len": [8],
             "global": [-3, 0, 1, 7, 8, 12], "local": [0, 0, 1, 7, 8, 8]},
        ],
    }
    for name, obj in (("tiny_causal_q0.json", g), ("tiny_window_scores.json", w),
                      ("localize_examples.json", loc)):
        with open(os.path.join(HERE, name), "w") as f:
            json.dump(obj, f, indent=1)
            f.write("\n")


if __name__ == "__main__":
    main()
