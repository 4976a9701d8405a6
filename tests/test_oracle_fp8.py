"""Pins for the oracle's OCP FP8 E4M3 codec: named codes of the specification, round trips,
PyTorch's float8_e4m3fn conversion, ties to even and saturation."""
import json
import os

import numpy as np
import torch

from oracle import fp8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_named_codes():
    with open(os.path.join(GOLDEN, "ocp_e4m3_codes.json")) as f:
        g = json.load(f)
    for c in g["codes"]:
        v = fp8.decode_code(c["code"])
        assert v == c["value"] and np.signbit(v) == np.signbit(c["value"])
        assert int(fp8.encode(np.float64(c["value"]))) == c["code"]
    for c in g["nan_codes"]:
        assert np.isnan(fp8.decode_code(c))


def test_round_trip_all_codes():
    for c in range(256):
        v = fp8.decode_code(c)
        if np.isnan(v):
            continue
        assert int(fp8.encode(np.float64(v))) == c


def test_matches_torch_in_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200_000) * s for s in (1e-3, 0.05, 1, 30, 200)]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(fp8.encode(x), ref)


def test_ties_go_to_even_code():
    # midpoints between neighbouring codes
    vals = np.array([fp8.decode_code(c) for c in range(0x7F)])
    mids = (vals[:-1] + vals[1:]) / 2
    codes = fp8.encode(mids)
    lo = np.arange(0x7E)
    expect = np.where(lo % 2 == 0, lo, lo + 1)
    np.testing.assert_array_equal(codes, expect)


def test_saturates():
    assert int(fp8.encode(np.float64(449.0))) == 0x7E
    assert int(fp8.encode(np.float64(1e6))) == 0x7E
    assert int(fp8.encode(np.float64(-1e6))) == 0xFE
    assert int(fp8.encode(np.float64(-1e-9))) == 0x80
