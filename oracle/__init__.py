"""CPU oracle for FlexPrefill (test infrastructure only; never on the product path)."""
from .flexprefill import *  # noqa: F401,F403
