"""Pins for the planner simulation (CPU only)."""
from oracle import planner
from tests._golden import load


def test_align128():
    assert [planner.align128(n) for n in (0, 1, 128, 129, 256)] == [0, 128, 128, 256, 256]


def test_worked_packing_example():
    g = load("planner_example.txt")
    T, K, D, F = g["T"], g["K"], g["D"], g["F"]
    full = [planner.dm_full_state_bytes(R, T, K, D, F) for R in g["worst_rank_R"]]
    keep = planner.align128(T * D * 2)
    flags, starts, tested = planner.decide(full, keep, g["capacity_28k"])
    assert tested[2] == g["L2_candidate"] and tested[2] <= g["capacity_28k"]
    assert tested[3] == g["L3_candidate"] and tested[3] > g["capacity_28k"]
    assert [int(f) for f in flags] == g["flags_28k"]
    flags24, _, _ = planner.decide(full, keep, g["capacity_24k"])
    assert int(flags24[2]) == g["flags_24k_L2"]


def test_decision_is_strict_inequality_and_rewinds():
    flags, starts, tested = planner.decide([100, 100], 10, 210)
    assert flags == [False, False] and starts == [0, 100]
    flags, starts, tested = planner.decide([100, 100], 10, 199)
    assert flags == [False, True]
    flags, _, _ = planner.decide([100, 100, 100], 0, 0)
    assert flags == [True, True, True]
