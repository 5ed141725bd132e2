"""Reader for the small text fixtures under tests/golden/."""

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read(name):
    """Parses a fixture: ``shape Q K D``, ``codebook q v...``, ``frame n key v... key v...``."""
    books = None
    frames = []
    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            line = raw.split("#", 1)[0].split()
            if not line:
                continue
            if line[0] == "shape":
                q, k, d = (int(v) for v in line[4:7])
                books = np.zeros((q, k, d), np.float32)
            elif line[0] == "codebook":
                q = int(line[1])
                books[q] = np.array([float(v) for v in line[2:]], np.float32).reshape(books.shape[1:])
            elif line[0] == "frame":
                rec, key = {}, None
                for tok in line[2:]:
                    try:
                        v = float(tok)
                    except ValueError:
                        key = tok
                        rec[key] = []
                        continue
                    rec[key].append(v)
                frames.append(rec)
    return books, frames
