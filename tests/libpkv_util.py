"""Locate / build libpkv.so for tests (builds only when nothing is built)."""

import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "paged_kv_cache_200_amd", "libpkv.so")


def ensure_built():
    if not os.path.exists(LIB):
        try:
            from paged_kv_cache_200_amd import build as b
            b.build()
        except Exception as e:  # no hipcc in this environment
            pytest.skip(f"libpkv.so not built and cannot be built here: {e}")
    return LIB
