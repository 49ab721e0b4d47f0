"""Hand-derived cache-append cases in tests/golden/append/ against the oracle
(CPU only).  Each fixture states the operation with the page and section
that define it and gives codes and scale worked out by hand."""
import glob
import os

import numpy as np
import pytest
import torch

from oracle import append_ref
import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "append")
FILES = sorted(glob.glob(os.path.join(GOLDEN, "*.txt")))


def _parse(path):
    kv = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    return kv


def test_fixtures_present():
    assert FILES


@pytest.mark.parametrize("path", FILES, ids=[os.path.basename(p) for p in FILES])
def test_oracle_quantizes_the_hand_derived_row(path):
    g = _parse(path)
    head = np.array([float(x) for x in g["row_head"].split()], np.float32)
    row = np.zeros(576, np.float32)
    row[:head.size] = head
    bits = torch.from_numpy(row).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.decode_bf16(bits), row.astype(np.float64)), "inputs must be bf16"
    want = np.array([int(x, 16) for x in g["codes_head"].split()], np.uint8)
    # the quantizer alone
    codes, scale = append_ref.quantize_rows_e4m3((bits.astype(np.uint32) << 16).view(np.float32))
    assert float(scale) == float(g["scale"])
    assert np.array_equal(codes[:want.size], want)
    assert np.all(codes[want.size:] == 0)
    # and through the append: one sequence of one page, the row as its 3rd token
    kv = np.full((2, 64, 576), 0x7F, np.uint8)
    sc = np.full((2, 64), np.nan, np.float32)
    bt = np.array([[1, 0]], np.int32)
    kv2, sc2, skipped = append_ref.kv_append_ref(kv, sc, bt, np.array([3], np.int32),
                                                 np.array([1], np.int32), bits[None, None, :],
                                                 64, "fp8_e4m3")
    assert skipped == 0
    assert np.array_equal(kv2[1, 2, :want.size], want) and float(sc2[1, 2]) == 2.0
    assert np.sum(kv2 != 0x7F) <= 576 and np.sum(~np.isnan(sc2)) == 1
