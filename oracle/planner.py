"""Saved-state byte accounting and the save/replay decision (test infrastructure).

Source: "Dist-MoE - Speed-of-light distributed Mixture-of-Experts kernels",
section 03 (align128(n) = ceil(n / 128) * 128; BF16 forward scratch
2R(D + 3F) bytes before alignment) and section 04 "Save and Recompute
Decisions": before saving a layer's full state the planner replays instead
when the worst rank's saved bytes plus that layer's full state, plus the
remaining layers times the bytes each must keep for replay, exceed the slot
capacity.  A replaying layer keeps only its replay input.  Backward runs the
layers in reverse and rewinds the cursor to each layer's start.

One GPU has one rank, so the worst-rank maximum is the value itself.
"""

from __future__ import annotations


def align128(n: int) -> int:
    return -(-int(n) // 128) * 128


def dm_full_state_bytes(R: int, T: int, K: int, D: int, F: int) -> int:
    """BF16 full state as the explainer counts it: gathered x [R,D], h1
    [R,2F] and the route-output slots [T*K, D], each aligned to 128 B."""
    return align128(R * D * 2) + align128(R * 2 * F * 2) + align128(T * K * D * 2)


def bf16_forward_scratch_bytes(R: int, D: int, F: int) -> int:
    """x_gathered, h1 and h2 of one call: 2R(D + 3F) bytes (before alignment)."""
    return 2 * R * (D + 3 * F)


def decide(full_bytes, keep_bytes: int, capacity: int):
    """Run the forward decisions of a stack of layers in one slot.

    ``full_bytes[l]`` is layer l's full saved state, ``keep_bytes`` what a
    replaying layer keeps (its replay input).  Returns (need_recompute list,
    start cursor of each layer, candidate value tested for each layer).
    Layer l replays iff cursor + full_l + (L - 1 - l) * keep > capacity; the
    cursor then advances by keep (replay) or full_l (save).
    """
    L = len(full_bytes)
    cursor = 0
    flags, starts, tested = [], [], []
    for l, full in enumerate(full_bytes):
        cand = cursor + int(full) + (L - 1 - l) * int(keep_bytes)
        starts.append(cursor)
        tested.append(cand)
        replay = cand > capacity
        flags.append(replay)
        cursor += int(keep_bytes) if replay else int(full)
    return flags, starts, tested


def bf16_full_state_bytes(R: int, D: int, F: int, es: int = 2) -> int:
    """This library's saved state of a BF16 (es = 2) or FP32 (es = 4) layer:
    h1 [R, 2F], aligned to 128 B.  Section 04 also lists the gathered x rows;
    on one GPU they are a copy of the caller's x, which the backward reads
    again through the permutation, and the route outputs h3 live in the
    caller's slot buffer.  (D is kept for the signature of the other byte
    terms.)"""
    return align128(R * 2 * F * es)


def mx_full_state_bytes(R: int, Rp: int, D: int, F: int) -> int:
    """This library's saved state of an MXFP8 layer (explainer section 04:
    MXFP8 full-save keeps the x and h2 column bundles and dense h1): x bundle
    codes [D, Rp] and exponents [D, Rp/32], BF16 h1 [R, 2F], h2 bundle codes
    [F, Rp] and exponents [F, Rp/32], each aligned to 128 B.  Rp = the rows
    padded to 32 per expert."""
    return (align128(D * Rp) + align128(D * Rp // 32) + align128(R * 2 * F * 2)
            + align128(F * Rp) + align128(F * Rp // 32))
