"""Runs every oracle pin against the oracle library named on the command line.

Used by tests/test_sanitizers.py to run the pins against a copy of oracle.c
built with AddressSanitizer and UndefinedBehaviorSanitizer (the interpreter
is started with the ASan runtime preloaded).  Prints "ok" when every pin
holds.
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
TESTS = os.path.dirname(HERE)
ROOT = os.path.dirname(TESTS)
for p in (ROOT, TESTS):
    if p not in sys.path:
        sys.path.insert(0, p)

import oracle  # noqa: E402
import _pins  # noqa: E402

o = oracle.Oracle(sys.argv[1])
for check in _pins.ALL_CHECKS:
    check(o)
    print("pin", check.__name__, "holds", flush=True)
print("ok")
