"""CPU oracle of the QuEST quantiser (test infrastructure only; see quest_oracle)."""
from .quest_oracle import *  # noqa: F401,F403
from .quest_oracle import __all__  # noqa: F401
