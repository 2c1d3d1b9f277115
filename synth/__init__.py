"""Seeded synthetic gradient sets shared by the tests, the smoke check and the
benchmark.  This module only draws random numbers and lays them out in the
storage formats; it holds none of the clipping arithmetic."""
from .gradsets import (GradSet, CONFIGS, make, shapes_tiny, shapes_andrea120m, shapes_gpt1p3b,
                       to_storage, storage_dtype)

__all__ = ["GradSet", "CONFIGS", "make", "shapes_tiny", "shapes_andrea120m", "shapes_gpt1p3b",
           "to_storage", "storage_dtype"]
