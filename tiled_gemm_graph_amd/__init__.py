"""MI355X persistent tile-graph megakernel.

A static graph of GEMMs with fused epilogues, RMSNorms, causal attention and
elementwise ops is compiled on the host (C++, libmk.so) into a flat list of
tile instructions with per-tile int32 dependency counters and executed by one
persistent HIP kernel per forward on gfx950.  See include/mk.h for the C ABI.
"""
from . import _lib
from ._lib import MkError
from .graph import Graph, Plan

__all__ = ["Graph", "Plan", "MkError", "load"]


def load():
    """Load libmk.so (raises ImportError if it has not been built)."""
    return _lib.load()
