"""Seeded synthetic workloads for the GDN state update (shared by tests, bench and smoke)."""
from .gen import *  # noqa: F401,F403
