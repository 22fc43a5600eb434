"""CPU oracle (test infrastructure only; see ``ae_oracle``)."""
from . import ae_oracle  # noqa: F401
