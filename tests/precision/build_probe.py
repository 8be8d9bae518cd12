"""Builds the test-only contraction probe (tests/precision/contraction_probe.hip)
into libcontraction_probe.so next to it, with the library's hipcc flags."""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "contraction_probe.hip")
LIB = os.path.join(HERE, "libcontraction_probe.so")


def build(verbose: bool = False) -> str:
    from sparse_attention_indexer_decode_amd._build import HIPCC_FLAGS, hipcc
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB
