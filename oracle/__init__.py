"""CPU oracle of the lockstep tick.  TEST INFRASTRUCTURE ONLY: imported by
tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg, never by the
GPU library."""
from .tick import Oracle, rmsnorm, silu, rope_interleaved, softmax_attend, greedy, upcast_bf16, round_bf16  # noqa: F401
