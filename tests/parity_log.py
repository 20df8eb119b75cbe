"""Collects the per-case figures of the GPU parity tests (errors, near-tie listings,
needle masses) so that a test session leaves a plain-text record of them.

conftest.py writes the collected lines when the session ends, to the path in the
LVQ_PARITY_RECORD environment variable, else to gpurun_out/parity_record.txt under
the repository root.  Imports nothing, so CPU-only sessions pay nothing for it.
"""
from __future__ import annotations

LINES: list[str] = []
_current = [""]


def case(name: str) -> None:
    """Starts the record of a test case; also printed, flushed, so a failing run names it."""
    _current[0] = name
    LINES.append(f"\n[{name}]")
    print(f"\ncase {name}", flush=True)


def line(text: str) -> None:
    LINES.append("  " + text)
    print("  " + text, flush=True)
