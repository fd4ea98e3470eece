"""Reader for the hand-written golden fixtures under tests/golden/."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_blocks(name):
    """Parse a fixture into {header: [row strings]} (comments and blanks skipped)."""
    blocks, cur = {}, None
    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            line = raw.strip()
            if not line or line.startswith("#"):
                continue
            if line[0].isalpha():
                cur = line
                blocks[cur] = []
            else:
                blocks[cur].append(line)
    return blocks


def mask_from_rows(rows):
    return np.array([[c == "1" for c in r] for r in rows], dtype=bool)
