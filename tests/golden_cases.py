"""Loader for tests/golden/oracle_cases.json (written by
tests/golden/make_oracle_cases.py from the CPU oracle alone)."""

import json
import os

import numpy as np

PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "oracle_cases.json")


def load():
    with open(PATH) as f:
        return json.load(f)["cases"]


def u16(h, shape):
    return np.frombuffer(bytes.fromhex(h), dtype=np.uint16).reshape(shape).copy()


def u8(h, shape):
    return np.frombuffer(bytes.fromhex(h), dtype=np.uint8).reshape(shape).copy()


def f32(h):
    return np.frombuffer(bytes.fromhex(h), dtype=np.float32)[0]


def qt_shapes(R, C, fmt):
    """Output shapes of a row + column quantization of x [R, C]."""
    w = 1 if fmt == "mxfp8" else 2
    b = 16 if fmt == "nvfp4" else 32
    return dict(row_codes=(R, C // w), row_scales=(R, C // b),
                col_codes=(C, R // w), col_scales=(C, R // b))


def ids(cases):
    return [c["name"] for c in cases]


def f32s(h):
    return np.frombuffer(bytes.fromhex(h), dtype=np.float32).copy()
