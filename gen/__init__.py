"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the benchmark."""
from .fields import WORKLOADS, Workload, make_dout, make_qkv, make_random_qkv, GENERATOR_VERSION  # noqa: F401
