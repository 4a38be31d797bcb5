"""Seeded synthetic inputs (shared by the oracle side and the GPU side; no layer arithmetic)."""
from .workloads import (FMT_BF16, FMT_F32, FMT_FP8, FMT_MX4, FMT_MX8, FMT_NV4, SIGMOID, SOFTMAX,
                        WORKLOADS, Workload)
from . import gen

__all__ = ["Workload", "WORKLOADS", "gen", "FMT_F32", "FMT_BF16", "FMT_FP8", "FMT_MX4",
           "FMT_MX8", "FMT_NV4", "SOFTMAX", "SIGMOID"]
