"""Loader for the hand-written fixtures in this folder (each cites its source)."""
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def load(name):
    """Parse a fixture into a list of (key, value-string) pairs, comments dropped."""
    items = []
    with open(os.path.join(HERE, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(" ")
            items.append((key, rest.strip()))
    return items


def hex_bytes(s):
    return np.frombuffer(bytes.fromhex(s.replace(" ", "")), np.uint8)


def floats(s):
    return np.array([float(v) for v in s.split()], np.float32)
