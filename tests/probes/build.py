"""Builds the fp32 operations probe (test infrastructure) with the library's flags."""

from __future__ import annotations

import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from sharded_flatparameter_flatten_amd import build as libbuild  # noqa: E402

PROBE = "libfp32probe.so"


def path() -> str:
    return os.path.join(HERE, PROBE)


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "fp32_ops_probe.hip")
    tmp = path() + ".tmp"
    libbuild._run([libbuild.HIPCC, "-x", "hip", *libbuild.DEVICE, *libbuild.COMMON, "-shared",
                   src, "-o", tmp], verbose)
    os.replace(tmp, path())
    return path()


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
