"""Synthetic workload shapes and seeded input generators (no method arithmetic)."""
