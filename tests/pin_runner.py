"""Run every oracle pin against one build of the oracle, in its own process.

Usage: python pin_runner.py LIBRARY_PATH
Prints one line per pin ("ok NAME" or "caught NAME") and exits 0.  A broken
copy of the oracle may also crash this process; the caller counts that as
caught too.
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
sys.path.insert(0, os.path.dirname(HERE))

import oracle          # noqa: E402
import oracle_pins     # noqa: E402


def main(path):
    o = oracle.Oracle(path)
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(o)
            print("ok", pin.__name__, flush=True)
        except AssertionError:
            print("caught", pin.__name__, flush=True)


if __name__ == "__main__":
    main(sys.argv[1])
