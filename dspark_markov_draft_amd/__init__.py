"""MI355X (gfx950) DSpark Markov draft walk: a C-ABI HIP library (libdspark.so, declared in
include/dspark.h) and its thin Python binding. Importing the package does not load the library;
the first call does, and raises if it is not built."""
from .binding import (  # noqa: F401
    BF16, F16, F32, DsparkError, check_workspace, dspark_debug_set, dspark_kernel_times,
    dspark_philox_words, dspark_quantize_w2, dspark_status_string, dspark_walk_greedy,
    dspark_walk_greedy_noalloc, dspark_walk_plan_query, dspark_walk_sample, dspark_walk_topk,
    dspark_walk_workspace_bytes, dspark_workspace_status, new_workspace, dspark_verify,
    dspark_verify_workspace_bytes, VERIFY_TOKEN, VERIFY_BLOCK, dspark_w2_prune_bound,
    dspark_walk_greedy_pruned, dspark_walk_sample_icdf,
)
