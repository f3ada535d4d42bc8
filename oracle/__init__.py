"""fp64 CPU oracle (test infrastructure only).

Only the tests, the smoke entry point and the benchmark's CPU-baseline leg
may import this package.  It shares no code with the HIP library.
"""
from .attention import (attention, chunk_bounds, merge_closed_form,  # noqa: F401
                        merge_fold, chunked_attention, ring_share, seq2head,
                        head2seq, ulysses_share, head_groups, groups_to_seq,
                        ulysses_anything_share, usp_share, usp_attention)
