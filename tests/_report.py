"""Measurement lines of the GPU tests (max and mean differences, bounds).

pytest captures what passing tests print, so each measurement is also kept
here and printed again, test by test, in a "parity measurements" section at
the end of the run (tests/conftest.py)."""
LINES = []


def report(msg: str) -> None:
    LINES.append(msg)
    print(f"[measure] {msg}", flush=True)
