"""CPU oracle for block-sparse attention (test infrastructure only; see
bsa_oracle's header).  Imports nothing from the product package."""
from . import bsa_oracle  # noqa: F401
