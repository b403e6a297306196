"""CPU oracle (test infrastructure only): see ``oracle.lsa_oracle``."""
from .lsa_oracle import *  # noqa: F401,F403
