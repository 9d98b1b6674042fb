"""Values the pages print, stored under tests/golden/ with their citation."""

import json
import os

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_mask_storage_bytes_at_128k():
    g = json.load(open(os.path.join(GOLDEN, "mask_storage_128k.json")))
    dense, vec = oracle.mask_storage_bytes(g["n"])
    assert dense == g["dense_bytes"]
    assert vec == g["vector_bytes"]
    assert dense // vec == g["ratio"]
