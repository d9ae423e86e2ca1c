"""Pins of the oracle's MX quantiser: hand examples from the OCP MX rule, every
E4M3 code against torch's float8_e4m3fn, and rounding against torch's cast."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import mx

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "mx_examples.json")))


def test_all_codes_decode_like_torch():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(mx.e4m3_decode(codes), ref)
    # encode(decode(c)) = c for every non-NaN code (round trip of representable values)
    np.testing.assert_array_equal(mx.e4m3_encode(mx.e4m3_decode(codes)), codes)


def test_encode_matches_torch_cast():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(20000) * s for s in (1e-4, 1e-2, 1, 30, 300)])
    v = np.clip(v, -448, 448)
    v = torch.tensor(v).to(torch.float32).to(torch.float64).numpy()
    ref = torch.tensor(v, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = mx.e4m3_encode(v)
    # torch keeps no sign on zero results of tiny negatives in all builds; compare magnitudes there
    zero = (ours & 0x7F) == 0
    np.testing.assert_array_equal(ours[~zero], ref[~zero])
    assert np.all((ref[zero] & 0x7F) == 0)


@pytest.mark.parametrize("ex", GOLD["elements"], ids=lambda e: e["why"])
def test_element_hand_examples(ex):
    assert int(mx.e4m3_encode(np.array([ex["value"]]))[0]) == ex["code"]


@pytest.mark.parametrize("blk", GOLD["blocks"], ids=lambda b: b["what"])
def test_block_hand_examples(blk):
    a = np.full((3, 64), blk["value"])
    c, s = mx.mx_quantize(a, axis=1)
    assert s.shape == (3, 2)
    assert np.all(s == blk["scale_code"]) and np.all(c == blk["elem_code"])
    np.testing.assert_array_equal(mx.mx_dequantize(c, s, axis=1), np.full_like(a, blk["dequant"]))


def test_block_scale_is_floor_log2_amax_minus_8_and_error_bound():
    rng = np.random.default_rng(1)
    a = rng.standard_normal((64, 96)) * np.exp(rng.uniform(-8, 8, size=(64, 1)))
    for axis in (0, 1):
        c, s = mx.mx_quantize(a, axis=axis)
        blocks = np.moveaxis(a, axis, -1).reshape(-1, 32)
        amax = np.abs(blocks).max(1)
        X = np.moveaxis(s, axis, -1).reshape(-1).astype(int) - 127
        assert np.all(2.0 ** (X + 8) <= amax) and np.all(amax < 2.0 ** (X + 9))
        dq = oracle.mx_roundtrip(a, axis=axis)
        # in scaled units v' = v / 2^X, a non-saturated element is within half an E4M3
        # ulp: 2^(floor(log2|v'|) - 4) for normals, 2^-10 below the smallest normal
        Xe = np.repeat(X.reshape(-1, 1), 32, axis=1)
        vs = blocks / 2.0 ** Xe
        err = np.abs(np.moveaxis(dq, axis, -1).reshape(-1, 32) - blocks) / 2.0 ** Xe
        e = np.floor(np.log2(np.maximum(np.abs(vs), 1e-300)))
        half_ulp = np.where(np.abs(vs) < 2.0 ** -6, 2.0 ** -10, 2.0 ** (e - 4))
        sat = np.abs(vs) > 448
        assert np.all(err[~sat] <= half_ulp[~sat])
        assert np.all(err[sat] == np.abs(vs[sat]) - 448)


def test_zero_padded_tail_and_quantise_axis():
    a = np.zeros((4, 32))
    a[1, 3] = 3.0
    with pytest.raises(ValueError):
        mx.mx_quantize(a, axis=0)          # 4 rows: not a whole block along axis 0
    c, s = mx.mx_quantize(np.concatenate([a, np.zeros((28, 32))]), axis=0)
    assert s.shape == (1, 32)
    assert s[0, 3] == 1 + 127 - 8 and c[1, 3] == mx.e4m3_encode(np.array([3.0 * 2 ** 7]))[0]
    assert s[0, 0] == 0 and np.all(c[:, 0] == 0)
    with pytest.raises(ValueError):
        mx.mx_quantize(np.zeros((5, 31)), axis=1)
