"""CPU oracle (test infrastructure only; never imported by the product path).

See ``oracle.prune24`` for the definitions it implements and their sources.
"""
from . import prune24  # noqa: F401
