"""The prefill GEMM's LDS ring schedule, simulated on the CPU.

The kernel (rotation_int4_weight_amd/csrc/prefill.hip) passes weight tiles
from producer waves to consumer waves through a ring of 8 LDS slots, with
workgroup barriers as the only ordering.  This model replays which tile each
role writes or reads between consecutive barriers and checks the three
conditions that make the ring race-free:
  * a slot is never written in the same barrier interval in which it is read;
  * a tile is read only after the barrier that follows its write;
  * between a tile's write and its last read, nothing else is written to its
    slot.
The numbers below restate the kernel's schedule: the producer expands tiles
0..4 before the first barrier, passes one extra barrier, then expands four
tiles (4S+5 .. 4S+8) per super-step S; the consumers read tile 0 between the
first two barriers and tiles 4S+1 .. 4S+4 during super-step S.  A persistent
workgroup numbers its steps across its output tiles, so several tiles are
one long schedule; between two output tiles the consumers run the epilogue,
which touches no ring slot, and they must read the next tile's first weight
tile during the last super-step of the previous one (not after the epilogue).
"""
import pytest

SLOTS = 8


def schedule(nsteps, extra_barrier=True, late_refill_every=0):
    """Lists of (interval, role, tile) events; interval i lies between
    barrier i-1 and barrier i (interval 0 precedes the first barrier)."""
    ev = []
    for t in range(5):
        ev.append((0, "w", t))
    first = 2 if extra_barrier else 1   # interval of super-step 0
    ev.append((1, "r", 0))
    for S in range(nsteps // 4):
        iv = first + S
        for u in range(4):
            ev.append((iv, "w", 4 * S + 5 + u))   # past the end too: clamped tiles still land in slots
            t = 4 * S + 1 + u
            if t >= nsteps:
                continue
            # late_refill_every = n: the first weight tile of every n-step
            # output tile read after the barrier ending the previous one
            late = late_refill_every and t % late_refill_every == 0
            ev.append((iv + 1 if late else iv, "r", t))
    return ev


def violations(ev):
    bad = []
    by_iv = {}
    for iv, role, t in ev:
        by_iv.setdefault(iv, []).append((role, t))
    for iv, items in by_iv.items():
        w = {t % SLOTS for r, t in items if r == "w"}
        r = {t % SLOTS for r_, t in items if r_ == "r"}
        if w & r:
            bad.append(f"interval {iv}: slot(s) {sorted(w & r)} written and read")
    writes = {}
    for iv, role, t in ev:
        if role == "w":
            writes.setdefault(t % SLOTS, []).append((iv, t))
    for iv, role, t in ev:
        if role != "r":
            continue
        wt = [(wi, tt) for wi, tt in writes[t % SLOTS] if tt == t]
        if not wt or wt[0][0] >= iv:
            bad.append(f"tile {t} read in interval {iv} before its write is ordered")
            continue
        later = [(wi, tt) for wi, tt in writes[t % SLOTS] if wi <= iv and tt != t and wi >= wt[0][0]]
        if later:
            bad.append(f"tile {t}'s slot overwritten by tile {later[0][1]} before its read in interval {iv}")
    return bad


@pytest.mark.parametrize("nsteps", [4, 8, 12, 16, 448])
def test_ring_schedule_is_race_free(nsteps):
    assert violations(schedule(nsteps)) == []


def test_model_detects_the_single_barrier_schedule():
    """Without the extra barrier, tile 8 lands in slot 0 while tile 0 is read."""
    bad = violations(schedule(8, extra_barrier=False))
    assert any("slot(s) [0]" in b for b in bad)


@pytest.mark.parametrize("tile_steps", [4, 8, 128])
def test_persistent_schedule_over_several_output_tiles(tile_steps):
    """Seven output tiles of tile_steps k steps each in one workgroup."""
    assert violations(schedule(7 * tile_steps)) == []


def test_model_detects_a_refill_after_the_epilogue():
    """Reading the next output tile's first weight tile after the barrier
    that ends the previous tile races with the producers' next super-step,
    which rewrites that slot."""
    assert any("slot(s)" in b for b in violations(schedule(7 * 8, late_refill_every=8)))
