"""Builds the fp32 operations probe (test infrastructure) with the library's flags."""

from __future__ import annotations

import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import importlib.util  # noqa: E402

# the library's build script, loaded by its path (importing it through the
# package would load the library itself)
_spec = importlib.util.spec_from_file_location(
    "fsdpshard_build", os.path.join(ROOT, "sharded_flatparameter_flatten_amd", "build.py"))
libbuild = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(libbuild)

PROBE = "libfp32probe.so"
STREAM_MIX = "libstreammix.so"


def path() -> str:
    return os.path.join(HERE, PROBE)


def stream_mix_path() -> str:
    return os.path.join(HERE, STREAM_MIX)


def _build_one(src_name: str, out: str, verbose: bool) -> str:
    tmp = out + ".tmp"
    libbuild._run([libbuild.HIPCC, "-x", "hip", *libbuild.DEVICE, *libbuild.COMMON, "-shared",
                   os.path.join(HERE, src_name), "-o", tmp], verbose)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Builds both probes; returns the fp32 probe's path."""
    _build_one("stream_mix_probe.hip", stream_mix_path(), verbose)
    return _build_one("fp32_ops_probe.hip", path(), verbose)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
