"""CPU fp64 oracle (test infrastructure only; see ``oracle.oracle``)."""
from .oracle import *  # noqa: F401,F403
from .oracle import (Decoded, decode_bf16, decode_e4m3, exact_topk, predict_paths,  # noqa: F401
                     predict_row, replay, sample_count, sample_positions, score_pairs,
                     score_row, select, select_from_candidates, threshold,
                     threshold_rank, expected_candidates, scoring_flops,
                     indexer_pairs, backward_query, backward_core, backward,
                     decode_e2m1, decode_e8m0, decode_mx)
