"""CPU fp64 oracle (test infrastructure only): see bd_oracle."""
from .bd_oracle import *  # noqa: F401,F403
