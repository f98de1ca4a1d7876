"""Lines the GPU parity tests record for the end-of-session summary (printed
by tests/conftest.py, so the class counts appear in a plain `pytest -q` run)."""

LINES = []


def record(line: str) -> None:
    LINES.append(line)
