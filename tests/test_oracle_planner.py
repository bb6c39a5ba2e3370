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


def test_mx_state_bytes_match_the_saved_tensors():
    """The MXFP8 saved-state formula equals the byte size of the tensors a
    full-save keeps (explainer section 04, MXFP8 full-save: x and h2 column
    bundles plus dense h1), built with the oracle's own quantizers on a tiny
    skewed layer where some experts are empty."""
    import numpy as np
    from mixture_experts_routed_03_amd import workloads as wl
    from oracle import moe as om
    from oracle import mx as omx
    T, D, F, E, K = 50, 64, 32, 7, 2
    ids, _ = wl.make_routing(T, E, K, zipf_s=1.5, n_pad=3, seed=2)
    rt = om.route(ids, E)
    rng = np.random.default_rng(0)
    xrows = rng.standard_normal((rt["R"], D))
    h2 = rng.standard_normal((rt["R"], F))
    xb, xe, hb, he = [], [], [], []
    for e in range(E):
        a, b = rt["offsets"][e], rt["offsets"][e + 1]
        if a == b:
            continue
        q, ex = omx.quantize_cols(xrows[a:b]); xb.append(q.size); xe.append(ex.size)
        q, ex = omx.quantize_cols(h2[a:b]); hb.append(q.size); he.append(ex.size)
    h1_bytes = rt["R"] * 2 * F * 2
    want = sum(planner.align128(n) for n in (sum(xb), sum(xe), h1_bytes, sum(hb), sum(he)))
    assert planner.mx_full_state_bytes(rt["R"], rt["poffsets"][-1], D, F) == want
    assert rt["poffsets"][-1] % 32 == 0 and rt["poffsets"][-1] >= rt["R"]


def test_bf16_state_bytes():
    """h1 [R, 2F] of the act dtype, rounded up to 128 B."""
    assert planner.bf16_full_state_bytes(3, 128, 128) == 1536
    assert planner.bf16_full_state_bytes(1, 128, 128, es=4) == 1024
    assert planner.bf16_full_state_bytes(1, 128, 8) == 128   # 32 B -> one 128-B line
