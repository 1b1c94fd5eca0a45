"""Child process for the planted-mistake tests: runs every oracle pin against a
mutant oracle library given on the command line.

Exit 0 when, for both the full-product and the per-element entry point, at
least one pin fails; exit 3 when some entry point passes every pin.
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import oracle  # noqa: E402
import test_oracle_pins as P  # noqa: E402


def main(path):
    lib = oracle.open_library(path)
    status = 0
    for entry, fn in (("full", P._full(lib)), ("at", P._at(lib))):
        failed = []
        for pin in P.ALL_PINS:
            try:
                if pin(fn):
                    failed.append(pin.__name__)
            except Exception as e:
                failed.append(f"{pin.__name__}:{type(e).__name__}")
        print(entry, "caught by", failed, flush=True)
        if not failed:
            status = 3
    return status


if __name__ == "__main__":
    sys.exit(main(sys.argv[1]))
