"""CPU oracle (test infrastructure only): the plain definition of the rotated low-bit
paged KV cache, used by the tests, the smoke check and the CPU baseline of the benchmark."""
from .kvq_oracle import *  # noqa: F401,F403
