"""Per-test parity counts of the GPU tests (sequences compared bit-exactly, near-ties
excluded, how many of those match anyway and how the rest were explained), gathered for
the terminal summary that tests/conftest.py prints at the end of the session."""

LINES = []


def add(line: str) -> None:
    LINES.append(line)
