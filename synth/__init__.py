"""Seeded synthetic workloads shared by the oracle-side and GPU-side tests and the bench."""
