"""Seeded synthetic inputs (no GEMM arithmetic) shared by tests, bench and oracle checks."""
