"""MI355X-native Medusa decode step: libmedusa (HIP/gfx950) and its Python binding.

The library is loaded lazily from the in-tree ``libmedusa.so``; importing this package
does not touch the GPU.  Build with ``python -m speculative_decoding_amd.build``.
"""
from . import medusa
from ._lib import LIB_PATH, header_functions, lib
from .medusa import MedusaError, TreePlan

__all__ = ["medusa", "lib", "LIB_PATH", "header_functions", "MedusaError", "TreePlan"]
