"""Run every oracle pin against one or more builds of the oracle.

Usage: python mutant_runner.py LIB.so [LIB.so ...]
Prints one JSON object: {lib path: [names of the pins that failed]}.
Used by test_oracle_mutants.py in a child process, so that a planted mistake
that crashes cannot take the test session down with it.
"""
import json
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import oracle  # noqa: E402
import pins  # noqa: E402


def main(libs):
    result = {}
    for lib in libs:
        oracle.use_library(lib)
        failed = []
        for pin in pins.ALL_PINS:
            try:
                pin()
            except (AssertionError, ValueError):
                failed.append(pin.__name__)
        result[lib] = failed
    oracle.use_library(None)
    print(json.dumps(result))


if __name__ == "__main__":
    main(sys.argv[1:])
