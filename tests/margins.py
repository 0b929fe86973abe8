"""Parity margins collected while the tests run, printed in the pytest
terminal summary (one line per case: the measured error, its bound, and the
ratio of the two)."""
from __future__ import annotations

RECORDS: list = []


def record(case: str, err: float, bound: float, what: str = "rel_err") -> None:
    RECORDS.append((case, what, float(err), float(bound)))
