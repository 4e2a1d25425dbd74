"""Hash of the attention kernels' code, so that counter readings taken on other
code are not reported as describing the current kernels.  Comments and layout
are left out: a reworded comment does not change what the counters measured."""
from __future__ import annotations

import hashlib
import os
import re

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
KERNEL_SOURCES = ("attn.hip", "common.hpp")


def code_text(src: str) -> str:
    """C++ source without comments and with whitespace collapsed: what the
    compiler sees (string literals in these sources hold no comment markers)."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()[:16]
