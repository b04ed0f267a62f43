"""Write random_kat.json: known-answer scores of the oracle's random draw.

Calls only the oracle.  Re-run (python tests/golden/make_random_kat.py) only
when the definition of the draw changes, and say why in the commit message.
"""

import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402

CASES = [
    (0, 0, 0, 0, 0, 0), (0, 0, 0, 0, 0, 1), (0, 0, 0, 0, 0, 2), (0, 0, 0, 0, 0, 3),
    (0, 0, 0, 0, 0, 4), (0, 0, 0, 1, 0, 5), (0, 0, 1, 0, 0, 5), (0, 1, 0, 0, 0, 5),
    (0, 0, 0, 0, 1, 5), (1, 0, 0, 0, 0, 5), (12345, 127, 35, 7, 29, 3135),
    (2**64 - 1, 2**32 - 1, 63, 15, 2**32 - 1, 2**31 - 1), (42, 3, 17, 2, 9, 1087),
]


def main():
    rows = []
    for seed, req, layer, head, rnd, i in CASES:
        u = oracle.random_draw(seed, req, layer, head, rnd, i)
        rows.append({"seed": seed, "request": req, "layer": layer, "head": head, "round": rnd,
                     "i": i, "u24": int(round(u * (1 << 24)))})
    with open(os.path.join(HERE, "random_kat.json"), "w") as f:
        json.dump({"_about": "oracle random draws, u = u24 / 2^24; written by make_random_kat.py",
                   "cases": rows}, f, indent=1)


if __name__ == "__main__":
    main()
