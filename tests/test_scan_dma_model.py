"""CPU model of the scan's DMA wave schedule (no GPU).

The DMA wave issues each chunk's loads in order (REC_KB record kilobytes,
then V_KB v kilobytes) into a ring of DEPTH LDS slots and waits with
explicit `s_waitcnt vmcnt(n)` counts: (DEPTH-1) x UNITS before the first
iteration (chunk 0 landed) and (DEPTH-2) x UNITS at the top of iteration c
(chunk c+1 landed).  Vector-memory loads of one wave complete in issue
order, so vmcnt(n) means "all but the last n issued have completed".  This
model replays the schedule for every column-part width the launch uses and
checks that each wait leaves exactly the chunk the compute waves read next
landed, that a slot is refilled only after the compute waves' reads of its
previous chunk (read one iteration ahead, before the barrier that ends the
iteration), and that the counts fit the 6-bit vmcnt field.
"""
from __future__ import annotations

import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "kimi_delta_attention_04_amd", "csrc")
SCAN_FILES = ("kda_scan_dev.h", "kda_scan.hip", "kda_bwd_scan.hip")


def scan_source() -> str:
    """The scan kernels' sources: the ring helpers, the forward scan and the
    backward's two scans."""
    return "\n".join(open(os.path.join(CSRC, f)).read() for f in SCAN_FILES)
REC_BYTES, CS = 13312, 16
VMCNT_MAX = 63


def ring_depth(cw: int) -> int:
    """RING_DEPTH<CW> of the source: 5 slots for parts of up to 64 columns, else 4."""
    return 5 if cw <= 64 else 4


def test_source_constants_match_model():
    src = scan_source()
    assert re.search(r"RING_DEPTH\s*=\s*CW\s*<=\s*64\s*\?\s*5\s*:\s*4", src)
    assert "wait_vm_barrier<(DEPTH - 1) * UNITS>()" in src
    assert "wait_vm_barrier<(DEPTH - 2) * UNITS>()" in src


@pytest.mark.parametrize("cw", [32, 64, 128])
@pytest.mark.parametrize("nch", [0, 1, 2, 3, 4, 5, 7, 64])
def test_dma_wait_ladder(cw, nch):
    rec_kb = REC_BYTES // 1024
    v_kb = CS * cw * 2 // 1024
    two_set_ladder(rec_kb + v_kb, ring_depth(cw), nch)


def two_set_ladder(units, depth, nch):
    """Replay of the two-operand-set protocol (see the module docstring)."""
    assert (depth - 1) * units <= VMCNT_MAX

    issued = []                      # chunk index of each issued load, in order
    completed = 0                    # loads completed (a prefix of `issued`)

    def issue(c):
        issued.extend([c] * units)

    def wait(n):
        nonlocal completed
        completed = max(completed, len(issued) - n)

    def landed(c):                   # every load of chunk c has completed
        return all(i < completed for i, x in enumerate(issued) if x == c)

    reads_done = set()               # chunks the compute waves have read into registers
    slot_of = {}

    for c in range(depth):           # prologue: fill the ring
        issue(c)
        slot_of[c] = c
    wait((depth - 1) * units)
    assert landed(0)
    reads_done.add(0)                # compute waves read chunk 0 after barrier B0
    slot = 0
    for c in range(nch):
        wait((depth - 2) * units)    # top of iteration c
        if c + 1 < nch + depth:
            assert landed(c + 1), (units, depth, nch, c)
        # barrier: the compute waves' reads of chunk c (issued in iteration
        # c-1) are complete; they now read chunk c+1
        assert c in reads_done
        reads_done.add(c + 1)
        # refill the slot chunk c occupied with chunk c + depth
        assert slot_of[c] == slot
        issue(c + depth)
        slot_of[c + depth] = slot
        # the slot being refilled holds no chunk the compute waves still need
        assert all(x <= c for x, s in slot_of.items() if s == slot and x != c + depth)
        slot = 0 if slot == depth - 1 else slot + 1
    wait(0)                          # the final drain
    assert completed == len(issued)


REC_BYTES_256 = 26624                # head dimension 256: 26 KB records


def test_wide_source_constants_match_model():
    src = scan_source()
    assert re.search(r"RING_DEPTH_256\s*=\s*4;", src)
    assert re.search(r"ONESET\s*=\s*WIDE\s*\|\|\s*CT\s*==\s*2;", src)
    assert "for (int c = 0; c < DEPTH - 1; ++c) issue(c, c);" in src
    assert "issue(c - 1 + DEPTH, slot);" in src


@pytest.mark.parametrize("rec_bytes,cw", [(REC_BYTES_256, 32), (REC_BYTES_256, 64),
                                          (REC_BYTES_256, 128),
                                          (REC_BYTES, 128)])
@pytest.mark.parametrize("nch", [0, 1, 2, 3, 4, 5, 7, 64])
def test_dma_wait_ladder_wide(rec_bytes, cw, nch):
    rec_kb = rec_bytes // 1024
    v_kb = CS * cw * 2 // 1024
    one_set_ladder(rec_kb + v_kb, 4, nch)


def one_set_ladder(units, depth, nch):
    """The one-operand-set protocol (256-wide tiles, and two slices per
    wave at 128): DEPTH-1 chunks issued before the first
    iteration; at the top of iteration c a wait of (DEPTH-2) x UNITS leaves
    chunk c landed; after the barrier the compute waves read chunk c (their
    reads of chunk c-1 completed before it) and the DMA wave refills chunk
    c-1's slot with chunk c-1+DEPTH."""
    assert (depth - 2) * units <= VMCNT_MAX

    issued, completed = [], 0
    slot_of = {}

    def issue(c, slot):
        issued.extend([c] * units)
        slot_of[c] = slot

    def wait(n):
        nonlocal completed
        completed = max(completed, len(issued) - n)

    def landed(c):
        return all(i < completed for i, x in enumerate(issued) if x == c)

    for c in range(depth - 1):
        issue(c, c)
    reading = None                   # chunk whose slot the compute waves read
    slot = depth - 1
    for c in range(nch):
        wait((depth - 2) * units)
        assert landed(c), (units, depth, nch, c)
        # barrier: reads of chunk c-1 are complete; the compute waves read chunk c
        reading = c
        assert slot_of[c] == c % depth
        assert slot == (c - 1) % depth
        # the slot refilled now holds chunk c-1 (done) or nothing yet
        holder = [x for x, s in slot_of.items() if s == slot]
        assert all(x <= c - 1 for x in holder) and reading not in holder
        issue(c - 1 + depth, slot)
        slot = 0 if slot == depth - 1 else slot + 1
    wait(0)
    assert completed == len(issued)


def bwd_ring_depth(units: int, lag: bool) -> int:
    """bwd_ring_depth<UNITS, LAG> of the backward's scans: as deep as the
    vmcnt field allows, at most 8 slots."""
    return min(8, VMCNT_MAX // units + (2 if lag else 1))


# (record bytes, column-part width, protocol) of every backward scan
# instance: the reverse scan's record is the forward layout (7, 13 or 26 KB
# at K = 64, 128, 256), the states scan's 5, 9 or 17 KB; "lag" with eight
# compute waves, "one" (one operand set) on the 256-wide tiles.
BWD_SCANS = [(13312, 32, "two"), (13312, 64, "two"), (13312, 128, "lag"),
             (7168, 32, "two"), (7168, 64, "two"),
             (26624, 32, "one"), (26624, 64, "one"),
             (9216, 32, "two"), (9216, 64, "two"), (9216, 128, "two"),
             (5120, 32, "two"), (5120, 64, "two"),
             (17408, 32, "one"), (17408, 64, "one")]


def test_lag_source_constants_match_model():
    src = scan_source()
    assert "constexpr bool ONESET = VD > HD;" in src
    assert "constexpr bool LAG = !ONESET && NW > 4;" in src
    assert "63 / UNITS + (LAG ? 2 : 1) > 8 ? 8 : 63 / UNITS + (LAG ? 2 : 1)" in src
    assert "constexpr int DEPTH = bwd_ring_depth<UNITS, LAG || ONESET>();" in src
    assert "constexpr int DEPTH = bwd_ring_depth<UNITS, ONESET>();" in src
    assert "wait_vm_barrier<(DEPTH - 3) * UNITS>()" in src
    assert "issue(c + DEPTH - 1, slot);" in src
    assert "issue(c - 1 + DEPTH, slot);" in src
    assert "const int widest = V > HD ? 64 : V;" in src


@pytest.mark.parametrize("rec_bytes,cw,proto", BWD_SCANS)
@pytest.mark.parametrize("nch", [0, 1, 2, 3, 4, 5, 7, 64])
def test_dma_wait_ladder_bwd(rec_bytes, cw, proto, nch):
    """The backward's scans: the two-operand-set ladder at their ring depths,
    the lagged one for eight compute waves, the one-set one at 256."""
    units = rec_bytes // 1024 + CS * cw * 2 // 1024
    depth = bwd_ring_depth(units, proto != "two")
    assert depth >= 4
    if proto == "lag":
        lag_ladder(units, depth, nch)
    elif proto == "one":
        one_set_ladder(units, depth, nch)
    else:
        two_set_ladder(units, depth, nch)


def lag_ladder(units, depth, nch):
    """The reverse scan's protocol with eight compute waves (128 columns):
    DEPTH-1 chunks issued before the first iteration and a wait of
    (DEPTH-2) x UNITS for chunk 0; at the top of iteration c a wait of
    (DEPTH-3) x UNITS leaves chunk c+1 landed; after the barrier the compute
    waves read chunk c+1's first operands and chunk c's update operands, and
    the DMA wave refills chunk c-1's slot with chunk c-1+DEPTH."""
    assert (depth - 2) * units <= VMCNT_MAX

    issued, completed = [], 0
    slot_of = {}

    def issue(c, slot):
        issued.extend([c] * units)
        slot_of[c] = slot

    def wait(n):
        nonlocal completed
        completed = max(completed, len(issued) - n)

    def landed(c):
        return all(i < completed for i, x in enumerate(issued) if x == c)

    for c in range(depth - 1):
        issue(c, c)
    wait((depth - 2) * units)
    assert landed(0)                 # the compute waves read chunk 0's first operands
    slot = depth - 1
    for c in range(nch):
        wait((depth - 3) * units)
        assert landed(c + 1), (nch, c)
        # barrier: the reads of chunk c-1 (update operands) and of chunk c
        # (first operands) are complete; now chunk c+1's first operands and
        # chunk c's update operands are read from their slots
        assert slot_of[c] == c % depth and slot_of[c + 1] == (c + 1) % depth
        assert slot == (c - 1) % depth
        holder = [x for x, s in slot_of.items() if s == slot]
        assert all(x <= c - 1 for x in holder)
        issue(c - 1 + depth, slot)
        slot = 0 if slot == depth - 1 else slot + 1
    wait(0)
    assert completed == len(issued)
