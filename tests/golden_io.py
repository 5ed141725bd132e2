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


def read_projected(name):
    """Parses a per-stage projected fixture: ``shape Q K D H``, then per stage
    ``codebook``, ``w_in``, ``b_in``, ``w_out``, ``b_out`` rows, then ``frame`` records.
    Returns ``(params dict of float32 arrays, frames)``."""
    p, frames = {}, []
    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            line = raw.split("#", 1)[0].split()
            if not line:
                continue
            if line[0] == "shape":
                q, k, d, h = (int(v) for v in line[5:9])
                p = {"books": np.zeros((q, k, d), np.float32), "w_in": np.zeros((q, d, h), np.float32),
                     "b_in": np.zeros((q, d), np.float32), "w_out": np.zeros((q, h, d), np.float32),
                     "b_out": np.zeros((q, h), np.float32)}
            elif line[0] in ("codebook", "w_in", "b_in", "w_out", "b_out"):
                key = "books" if line[0] == "codebook" else line[0]
                q = int(line[1])
                p[key][q] = np.array([float(v) for v in line[2:]], np.float32).reshape(p[key].shape[1:])
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
    return p, frames
