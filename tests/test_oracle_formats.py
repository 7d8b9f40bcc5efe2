"""Pins of the oracle's FP4 / E4M3 decoders (CPU only).

E4M3 is checked code by code against torch's float8_e4m3fn -> float32 cast (an
independent library routine); E2M1 against the value fixture in
tests/golden/e2m1_values.txt; the nibble packing against hand-built rows."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import formats


def test_e4m3_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).double().numpy()
    for c in range(256):
        mine = formats.e4m3_value(c)
        if math.isnan(ref[c]):
            assert math.isnan(mine), c
        else:
            assert mine == ref[c], (c, mine, ref[c])
            assert math.copysign(1.0, mine) == math.copysign(1.0, ref[c]), c


def test_e4m3_special_values():
    assert formats.e4m3_value(0x7E) == 448.0
    assert formats.e4m3_value(0x01) == 2.0 ** -9          # smallest subnormal
    assert formats.e4m3_value(0x07) == 7 * 2.0 ** -9      # largest subnormal
    assert formats.e4m3_value(0x08) == 2.0 ** -6          # smallest normal
    assert formats.e4m3_value(0x38) == 1.0
    assert math.isnan(formats.e4m3_value(0x7F)) and math.isnan(formats.e4m3_value(0xFF))
    # 127 non-negative finite codes, strictly increasing
    g = formats.E4M3_GRID
    assert len(g) == 127 and np.all(np.diff(g) > 0) and g[0] == 0.0


def test_e2m1_matches_golden(golden_dir):
    rows = [ln.split() for ln in open(os.path.join(golden_dir, "e2m1_values.txt"))
            if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 16
    for code, val in rows:
        v = float(val)
        mine = formats.e2m1_value(int(code))
        assert mine == v and math.copysign(1, mine) == math.copysign(1, v), code


def test_constants_fixture(golden_dir):
    c = json.load(open(os.path.join(golden_dir, "csa2_constants.json")))
    assert c["pool_blocks"]["value"] * c["block_tokens"]["value"] == c["pool_positions"]["value"]
    assert formats.E4M3_MAX == c["e4m3_max"]["value"]
    # 437x: 389,000 / 890 rounds to 437
    assert round(c["v1_bytes_per_token"]["value"] / c["bytes_per_token_global_kv"]["value"]) == \
        c["reduction_vs_v1"]["value"]
    from oracle import indexer
    assert indexer.TOPK == c["topk"]["value"]
    assert indexer.BLOCK == c["block_tokens"]["value"]
    assert indexer.POOL_BLOCKS == c["pool_blocks"]["value"]


def test_dequant_rows_nibble_order_and_scale():
    # channel c of row 0 holds code c % 16; scales 1.0 (0x38) and 0.5 (0x30)
    dim = 32
    nib = np.arange(dim) % 16
    codes = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)[None, :]
    scales = np.array([[0x38, 0x30]], dtype=np.uint8)
    got = formats.dequant_rows(codes, scales, dim)[0]
    want = np.array([formats.e2m1_value(int(n)) for n in nib]) * np.repeat([1.0, 0.5], 16)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("dim", [128, 512])
def test_entry_bytes(dim):
    # d/2 code bytes + d/16 scale bytes per entry: 288 B at d = 512
    assert dim // 2 + dim // 16 == {128: 72, 512: 288}[dim]
