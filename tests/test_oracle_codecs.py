"""Pins for the oracle's stored-format decoders (CPU only).

bf16 and e4m3fn decoding are checked against torch's own dtype casts over
every bit pattern (a library routine independent of the oracle's table), and
against the format's fixed points.
"""
import math

import numpy as np
import pytest
import torch

from oracle import codecs

pytestmark = pytest.mark.filterwarnings("ignore")


def test_bf16_all_patterns_match_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = codecs.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_e4m3fn_table_matches_torch_cast():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = codecs.E4M3FN_TABLE
    nan = np.isnan(ref)
    assert nan.sum() == 2  # S.1111.111 for both signs
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_e4m3fn_format_facts():
    t = codecs.E4M3FN_TABLE
    assert np.nanmax(t) == 448.0 and np.nanmin(t) == -448.0
    assert t[1] == 2.0 ** -9                  # smallest subnormal
    assert t[0x08] == 2.0 ** -6               # smallest normal
    assert t[0x38] == 1.0                     # e=7 (bias), m=0
    assert t[0x80] == 0.0 and math.copysign(1, t[0x80]) < 0
    assert math.isnan(t[0x7F]) and math.isnan(t[0xFF])
    finite = t[~np.isnan(t)]
    assert len(np.unique(finite)) == 253      # +0/-0 compare equal


def test_e4m3_scale_applies_per_row():
    codes = np.array([[0x38, 0x40], [0x38, 0xB8]], dtype=np.uint8)   # 1, 2 ; 1, -1
    scale = np.array([0.5, 3.0], dtype=np.float32)
    v = codecs.e4m3_to_f64(codes, scale)
    assert np.array_equal(v, np.array([[0.5, 1.0], [3.0, -3.0]]))


def test_decode_rows_dispatch():
    assert codecs.decode_rows(np.array([[0x3F80]], dtype=np.uint16))[0, 0] == 1.0
    with pytest.raises(TypeError):
        codecs.decode_rows(np.zeros((1, 1), np.float32))
