"""Seeded synthetic inputs shared by the oracle side and the HIP side of every check.

Holds random draws and storage casts only (library casts to bfloat16 and
float8_e4m3fn); none of the mixer's arithmetic lives here.
"""
from .synthetic import *  # noqa: F401,F403
