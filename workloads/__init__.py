"""Seeded synthetic inputs shared by the HIP library's tests/bench and the CPU oracle."""
from .configs import Workload, WORKLOADS, BENCH_DEFAULT
from .generate import DSAInputs, generate, raw_numpy, dtype_tag, to_device

__all__ = ["Workload", "WORKLOADS", "BENCH_DEFAULT", "DSAInputs", "generate", "raw_numpy",
           "dtype_tag", "to_device"]
