"""CPU oracle (test infrastructure only; see woq_oracle's header)."""
from .woq_oracle import *  # noqa: F401,F403
from .woq_oracle import __doc__ as _doc  # noqa: F401
