"""Seeded synthetic workloads shared by the tests, the bench and the oracle checks."""
