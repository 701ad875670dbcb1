"""CPU oracle for the causal Self-Exchange Relation: test infrastructure only.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package; the product path never does.
"""
from .relation_oracle import *  # noqa: F401,F403
