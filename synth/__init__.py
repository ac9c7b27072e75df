"""Seeded synthetic inputs shared by the oracle's and the GPU library's tests
and by the benchmark, plus the benchmark's HBM bandwidth probes.  Holds no
attention arithmetic."""
