"""Builds the test-only probes (tests/precision/contraction_probe.hip and
mx_scale_probe.hip) into libcontraction_probe.so and libmx_scale_probe.so
next to them, with the library's hipcc flags."""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
PROBES = ("contraction_probe", "mx_scale_probe")
LIB = os.path.join(HERE, "libcontraction_probe.so")
MX_LIB = os.path.join(HERE, "libmx_scale_probe.so")


def build(verbose: bool = False) -> str:
    from sparse_attention_indexer_decode_amd._build import HIPCC_FLAGS, hipcc
    for name in PROBES:
        src = os.path.join(HERE, name + ".hip")
        lib = os.path.join(HERE, "lib" + name + ".so")
        tmp = lib + ".tmp"
        cmd = [hipcc(), *HIPCC_FLAGS, src, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
        os.replace(tmp, lib)
    return LIB
