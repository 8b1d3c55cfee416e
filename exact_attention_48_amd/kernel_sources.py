"""Which source files make up each kernel, and a short hash of them.

A committed HBM-traffic summary under ``profiles/`` records the hash of its
kernel's sources; a reader (``bench.py``) trusts the figure only while the hash
still matches, i.e. while the kernel has not changed since the counters were
taken.
"""
from __future__ import annotations

import hashlib
import os

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


def source_hash(kernel: str) -> str:
    """First 16 hex digits of the SHA-256 over the kernel's source files, in order."""
    h = hashlib.sha256()
    for n in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, n), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]
