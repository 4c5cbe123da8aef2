"""Writes zen_fig10.json: a hash seed under which the Fig. 10 walk-through of
the Zen page (section 3.3.2) can be replayed with the oracle's own h0.

The page's example: |G| = 15 indices, 3 servers; server 0's class I_0 holds the
two nonzero indices {5, 7} as its 2nd and 3rd members (indices counted from 1),
so the hash bitmap has its 2nd and 3rd bits set and decodes back to {5, 7}.
The page does not print the full I_0, so any h0 seed that makes 5 and 7 the
2nd and 3rd members of I_0 replays the example.  This build numbers indices
and bits from 0, so page index i is index i-1 here and page bit b is bit b-1.
Calls only the oracle.
"""
import json
import os
import sys

sys.path.insert(0, os.path.abspath(os.path.join(os.path.dirname(__file__), "..", "..")))
import oracle  # noqa: E402


def main():
    G, servers = 15, 3
    page_nonzero = [5, 7]
    zero_based = [i - 1 for i in page_nonzero]
    for seed in range(1, 1 << 20):
        c0 = [i for i in range(G) if oracle.h0(i, seed, servers) == 0]
        if all(x in c0 for x in zero_based) and c0.index(zero_based[0]) == 1 and c0.index(zero_based[1]) == 2:
            break
    doc = {
        "source": "Zen (OSDI'25) digest page, section 3.3.2 (hash bitmap), Fig. 10 walk-through",
        "G": G, "servers": servers, "seed": seed,
        "page_nonzero_indices_1based": page_nonzero,
        "page_set_bits_1based": [2, 3],
        "class0_0based": c0,
    }
    with open(os.path.join(os.path.dirname(__file__), "zen_fig10.json"), "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
