"""The sigmoid table the BF16 kernels read is generated at build time
(csrc/gen_sig_table.cpp writes csrc/sig_table.inc).  CPU check: every entry
equals the oracle's correctly rounded sigmoid of its BF16 pattern, and the
clamped ends of the pattern range round to the table's end values."""
import os
import re

import numpy as np
import pytest

from oracle import route_sort as orc

INC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "align_moe_route_amd", "csrc", "sig_table.inc")


def _table():
    if not os.path.exists(INC):
        pytest.skip("sig_table.inc is made by the build (__graft_entry__.build())")
    vals = re.findall(r"0x([0-9a-f]{8})u", open(INC).read())
    return np.array([int(v, 16) for v in vals], dtype=np.uint32).view(np.float32)


def test_generated_table_equals_oracle():
    tab = _table()
    assert tab.size == 8192
    t = np.arange(8192) & 4095
    s = np.arange(8192) >> 12
    h = (((0x3300 + t) & 0x7FFF) | (s << 15)).astype(np.uint16)
    ref = orc.sigmoid_f32(orc.bf16_bits_to_f32(h))
    bad = np.flatnonzero(tab.view(np.uint32) != ref.view(np.uint32))
    assert bad.size == 0, (h[bad[:5]], tab[bad[:5]], ref[bad[:5]])


def test_clamping_outside_the_table_is_exact():
    # below the first pattern every magnitude rounds to 1/2, from the last one
    # up the sigmoid is 1 (positive) or its value at the clamp pattern is the
    # same FP32 number as at every larger magnitude (negative)
    tab = _table()
    small = orc.bf16_bits_to_f32(np.arange(0, 0x3300, dtype=np.uint16))
    assert np.all(orc.sigmoid_f32(small) == np.float32(0.5))
    assert np.all(orc.sigmoid_f32(-small) == np.float32(0.5))
    big = orc.bf16_bits_to_f32(np.arange(0x4300 - 1, 0x7F80, dtype=np.uint16))
    assert np.all(orc.sigmoid_f32(big) == tab[4095])
    assert np.all(orc.sigmoid_f32(-big) == tab[4096 + 4095])
