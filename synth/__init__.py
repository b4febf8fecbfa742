"""Seeded synthetic input generators shared by tests, smoke check and benchmark."""
