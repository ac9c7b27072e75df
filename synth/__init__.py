"""Seeded synthetic inputs shared by the oracle's and the GPU library's tests
and by the benchmark.  Draws numbers only; holds no attention arithmetic."""
