"""Readers for the hand-written fixtures under tests/golden/."""

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _num(v):
    if isinstance(v, str):
        return -0.0 if v == "-0" else float(v)
    return float(v)


def _code(v):
    return int(v, 16) if isinstance(v, str) else int(v)


def load_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b = line.split()
            rows.append((a, b))
    return rows


def load_case(name):
    with open(os.path.join(GOLDEN, name)) as f:
        raw = json.load(f)
    case = dict(raw)
    case["W"] = np.array([[_num(v) for v in r] for r in raw["W"]], dtype=np.float32)
    case["x"] = np.array([[_num(v) for v in r] for r in raw["x"]], dtype=np.float16)
    case["y"] = np.array(raw["y"], dtype=np.float64)
    case["codes"] = np.array([[_code(v) for v in r] for r in raw["codes"]], dtype=np.uint8)
    if "block_scale_codes" in raw:
        case["block_scale_codes"] = np.array([[_code(v) for v in r] for r in raw["block_scale_codes"]], dtype=np.uint8)
        case["packed_codes"] = np.array([[_code(v) for v in r] for r in raw["packed_codes"]], dtype=np.uint8)
        case["dequantized"] = np.array([[_num(v) for v in r] for r in raw["dequantized"]], dtype=np.float64)
    if "row_scales" in raw:
        case["row_scales"] = np.array(raw["row_scales"], dtype=np.float32)
    return case
