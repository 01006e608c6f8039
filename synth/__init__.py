"""Seeded synthetic input generators (no layer arithmetic)."""
