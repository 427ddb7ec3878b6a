"""Lines that tests want in the run's summary (printed by conftest at the end of the
session, also under -q): whole-tensor parity numbers of the full-size workloads."""

LINES = []


def report(line: str) -> None:
    LINES.append(line)
