"""CPU oracle of the SPA-Cache layer step. Test infrastructure only: see spacache_oracle."""
from .spacache_oracle import *  # noqa: F401,F403
from .spacache_oracle import identify  # noqa: F401
