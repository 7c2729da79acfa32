"""Seeded synthetic inputs (no quantizer arithmetic)."""
