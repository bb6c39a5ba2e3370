"""Pins for the oracle's routing metadata (CPU only)."""
import itertools

import numpy as np
import pytest

from oracle import moe
from tests._golden import load


def test_scan_worked_example():
    g = load("scan_example.txt")
    counts = g["counts"]
    # Routes in scrambled expert order; the offsets only depend on the counts.
    ids = np.array(sum(([e] * c for e, c in enumerate(counts)), []))
    rng = np.random.default_rng(0)
    ids = ids[rng.permutation(ids.size)].reshape(-1, 1)
    rt = moe.route(ids, E=len(counts))
    assert rt["counts"].tolist() == counts
    assert rt["offsets"].tolist() == g["offsets"]


def _check_grouping(ids, E, rt):
    flat = ids.reshape(-1)
    valid = [r for r in range(flat.size) if 0 <= flat[r] < E]
    sr = rt["sorted_route"].tolist()
    # A permutation of the valid routes ...
    assert sorted(sr) == valid
    # ... expert-major with ascending route inside an expert (stable order).
    keys = [(int(flat[r]), r) for r in sr]
    assert keys == sorted(keys)
    hist = [sum(1 for r in valid if flat[r] == e) for e in range(E)]
    assert rt["counts"].tolist() == hist
    assert rt["offsets"][-1] == len(valid) == sum(hist)
    for e in range(E):
        a, b = rt["offsets"][e], rt["offsets"][e + 1]
        assert all(flat[r] == e for r in sr[a:b])
    inv = rt["route_to_row"]
    for row, r in enumerate(sr):
        assert inv[r] == row
    for r in range(flat.size):
        if r not in valid:
            assert inv[r] == -1
    pc = rt["poffsets"]
    for e in range(E):
        span = pc[e + 1] - pc[e]
        assert span % 32 == 0 and hist[e] <= span < hist[e] + 32


@pytest.mark.parametrize("T,K", [(1, 1), (2, 1), (1, 2), (3, 2), (2, 3), (6, 1)])
@pytest.mark.parametrize("E", [1, 2, 3])
def test_bruteforce_all_id_arrays(T, K, E):
    for combo in itertools.product(range(-1, E), repeat=T * K):
        ids = np.array(combo).reshape(T, K)
        rt = moe.route(ids, E)
        assert not rt["bad_id"]
        _check_grouping(ids, E, rt)


def test_bad_ids_flagged_and_treated_as_padding():
    ids = np.array([[0, 5], [-2, 1], [-1, 1]])
    rt = moe.route(ids, E=2)
    assert rt["bad_id"]
    assert rt["counts"].tolist() == [1, 2]
    assert rt["sorted_route"].tolist() == [0, 3, 5]
    assert rt["route_to_row"].tolist() == [0, -1, -1, 1, -1, 2]


def test_empty_and_all_padding():
    rt = moe.route(np.zeros((0, 3), dtype=np.int32), E=4)
    assert rt["R"] == 0 and rt["offsets"].tolist() == [0] * 5
    rt = moe.route(np.full((5, 2), -1), E=4)
    assert rt["R"] == 0 and rt["route_to_row"].tolist() == [-1] * 10


def test_slot_layout_worked_example():
    """Route output slot (t, k) sits at (t*K + k) * D * bytes from the combine
    base; the source row of token t at t * D * bytes."""
    g = load("slot_example.txt")
    r = g["t"] * g["K"] + g["k"]
    assert r * g["D"] * g["bytes_per_elem"] == g["slot_offset_bytes"]
    assert g["t"] * g["D"] * g["bytes_per_elem"] == g["source_offset_bytes"]
