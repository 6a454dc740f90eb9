"""Shared-memory / LDS bank-conflict simulator (TEST INFRASTRUCTURE ONLY).

Model (the bank arithmetic of "Swizzling explained properly", section "Why
swizzle?", and of "Tensor Cores, layouts, and swizzling", the bank-collision
paragraph): memory is split into ``nbanks`` banks of ``bank_bytes`` bytes;
byte address x lies in bank ``(x // bank_bytes) % nbanks``; a bank serves one
word per cycle, and lanes that read the *same* word share it.  A wide access
is serviced in phases (groups of lanes handled together); the swizzling page's
store analysis shows that a warp's 256-byte store is split into two 128-byte
transactions, i.e. two phases of 16 lanes.

For one instruction the simulator returns, per phase, the degree = the
largest number of distinct words any single bank must deliver.  Degree 1 is
conflict-free; the extra cycles of the instruction are sum(degree - 1).
"""
from __future__ import annotations

from typing import Iterable, List, Optional, Sequence


def consecutive_phases(nlanes: int, lanes_per_phase: int) -> List[List[int]]:
    return [list(range(s, min(s + lanes_per_phase, nlanes)))
            for s in range(0, nlanes, lanes_per_phase)]


def phase_degrees(addrs: Sequence[Optional[int]], width: int, nbanks: int = 32,
                  bank_bytes: int = 4,
                  phases: Optional[Iterable[Sequence[int]]] = None,
                  lanes_per_phase: Optional[int] = None) -> List[int]:
    """Degree of each phase of one access.

    addrs: byte address per lane (None = inactive lane); width: bytes each
    lane accesses (a multiple of bank_bytes, aligned).  Phases default to
    consecutive lanes, as many as fill one bank line
    (nbanks*bank_bytes // width), unless ``lanes_per_phase`` is given."""
    n = len(addrs)
    if phases is None:
        lpp = lanes_per_phase or max(1, (nbanks * bank_bytes) // width)
        phases = consecutive_phases(n, lpp)
    degrees = []
    for ph in phases:
        words_per_bank = {}
        for lane in ph:
            a = addrs[lane]
            if a is None:
                continue
            for w in range(a // bank_bytes, (a + width - 1) // bank_bytes + 1):
                words_per_bank.setdefault(w % nbanks, set()).add(w)
        degrees.append(max((len(s) for s in words_per_bank.values()), default=0))
    return degrees


def conflict_degree(*args, **kw) -> int:
    """Worst phase degree of one access (1 = conflict-free)."""
    return max(phase_degrees(*args, **kw), default=0)


def extra_cycles(*args, **kw) -> int:
    """Cycles lost to conflicts: sum over phases of (degree - 1)."""
    return sum(max(d - 1, 0) for d in phase_degrees(*args, **kw))
