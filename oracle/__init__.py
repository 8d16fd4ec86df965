"""CPU oracle of the nanochat-style GPT training step -- TEST INFRASTRUCTURE.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package.  The HIP library never loads it and it never loads the
HIP library.
"""
from .oracle import *  # noqa: F401,F403
