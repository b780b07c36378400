"""Parity counts that the GPU tests report (edge-band elements, forgiven
level mismatches, largest errors, bit-exact tokens).  The session's summary
prints them at the end of the run, one JSON line per case."""

from __future__ import annotations

RECORDS: list = []


def record(case: str, **counts) -> None:
    RECORDS.append((case, counts))
