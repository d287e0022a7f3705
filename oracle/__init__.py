"""CPU oracle (test infrastructure only; see qwen2_oracle's header)."""
from .qwen2_oracle import *  # noqa: F401,F403
from .qwen2_oracle import __all__  # noqa: F401
