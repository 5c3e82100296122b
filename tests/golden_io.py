"""Reader for the hand-derived fixtures under tests/golden/ (text, one case each)."""
from __future__ import annotations

import glob
import os

import numpy as np

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(path):
    case = {"name": os.path.splitext(os.path.basename(path))[0], "expect": {}}
    times, types = [], []
    in_events = False
    with open(path) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            if in_events:
                t, y = line.split()
                times.append(int(t))
                types.append(int(y))
                continue
            key, *vals = line.split()
            if key == "events":
                in_events = True
            elif key == "nodes":
                case["N"] = int(vals[0])
            elif key == "types":
                case["ep_types"] = np.array([int(v) for v in vals], dtype=np.uint16)
            elif key == "intervals":
                v = [int(x) for x in vals]
                case["t_low"] = np.array(v[0::2], dtype=np.int32)
                case["t_high"] = np.array(v[1::2], dtype=np.int32)
            elif key == "cut":
                case["cut"] = int(vals[0])
            elif key == "expect":
                case["expect"][vals[0]] = [int(x) for x in vals[1:]]
            else:
                raise ValueError("unknown key %r in %s" % (key, path))
    case["times"] = np.array(times, dtype=np.int32)
    case["types"] = np.array(types, dtype=np.uint16)
    if "t_low" not in case:
        case["t_low"] = np.zeros(0, dtype=np.int32)
        case["t_high"] = np.zeros(0, dtype=np.int32)
    assert len(case["ep_types"]) == case["N"]
    assert len(case["t_low"]) == case["N"] - 1
    return case


def all_cases():
    return [load(p) for p in sorted(glob.glob(os.path.join(GOLDEN_DIR, "*.txt")))]
