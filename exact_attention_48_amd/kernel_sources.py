"""Which source files make up each kernel, and a short hash of them.

A committed HBM-traffic summary under ``profiles/`` records the hash of its
kernel's sources; a reader (``bench.py``) trusts the figure only while the hash
still matches, i.e. while the kernel has not changed since the counters were
taken. The hash covers the code only: comments are removed and runs of
whitespace collapsed first, so editing a comment keeps a measurement valid.
"""
from __future__ import annotations

import hashlib
import os
import re

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")

_COMMON = ["fa_device.h", "fa_kernels.h", "fa_order.h", "fa_tiles.h"]

KERNEL_SOURCES = {
    "fa_fwd_pp_kernel": ["fa_fwd_pp.hip"] + _COMMON,
    "fa_fwd_kernel": ["fa_fwd.hip"] + _COMMON,
    "bwd_dkdv_kernel": ["fa_bwd.hip"] + _COMMON,
    "bwd_dq_kernel": ["fa_bwd.hip"] + _COMMON,
    "bwd_prep_kernel": ["fa_bwd.hip"] + _COMMON,
    "merge_kernel": ["fa_merge.hip"] + _COMMON,
}


def code_only(text: str) -> str:
    """C/C++ source without its comments, whitespace runs collapsed to one space.
    String and character literals are kept as written (a "//" inside one is code)."""
    out = []
    i, n = 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return re.sub(r"\s+", " ", "".join(out)).strip()


def source_hash(kernel: str) -> str:
    """First 16 hex digits of the SHA-256 over the code of the kernel's source files, in order."""
    h = hashlib.sha256()
    for n in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, n), encoding="utf-8") as fh:
            h.update(code_only(fh.read()).encode())
            h.update(b"\0")
    return h.hexdigest()[:16]
