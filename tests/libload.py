"""Locate the built HIP library for the tests (building it only if absent)."""

import os

from kv_cache_management_amd import build as B


def ensure_built() -> str:
    if not os.path.exists(B.LIB):
        B.build(verbose=False)
    return B.LIB
