"""CPU oracle for MassAlloc Attention (MALA): plain numpy float64.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the HIP library never does,
and the two share no code.
"""
from .mala_ref import *  # noqa: F401,F403
from .mala_ref import (BlockResult, backward_tile_grads, combine_split_rows, combine_splits,  # noqa: F401
                       post_score_slots, prefill_block_args, split_ranges)
