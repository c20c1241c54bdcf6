"""The oracle against the stored fixtures in tests/golden/.

* ``nibble_order.txt``: the packing rule's worked example (even element in the
  low nibble).
* ``tiny_oracle_digest.json``: written by ``tests/golden/make_golden.py`` from
  the oracle alone; guards the oracle's arithmetic against silent change.
"""
import json
import os

import numpy as np

import oracle as O
from tests.golden.make_golden import tiny_digests

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_nibble_order_fixture():
    lines = [l.split() for l in open(os.path.join(GOLDEN, "nibble_order.txt")) if l.strip() and not l.startswith("#")]
    for codes, bytes_ in zip(lines[0::2], lines[1::2]):
        assert codes[0] == "codes" and bytes_[0] == "bytes"
        c = np.array([int(v) for v in codes[1:]], np.uint8)
        assert O.pack_codes(c).tolist() == [int(v, 16) for v in bytes_[1:]]


def test_tiny_digest_fixture():
    stored = json.load(open(os.path.join(GOLDEN, "tiny_oracle_digest.json")))["digests"]
    assert tiny_digests() == stored
