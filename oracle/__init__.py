"""CPU fp64 oracle for the local Softmax branch of VDN-H3 hybrid video attention
(forward and backward), the complement linear branch and the fusion.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP path.

Pinned functions (each checked in the CPU test suite against something other
than itself: brute force, a library routine, closed forms, hand-derived
values from the pages' description):

* ``key_intervals`` / ``query_blocks``   -- brute-force mask scan, hand-derived
                                            interval lists
* ``allowed_mask``                       -- hand-picked pairs from the pages' rule
* ``count_pairs``                        -- brute-force mask count
* ``attend``                             -- dense masked attention, torch SDPA
                                            (float64) in the full-window case,
                                            closed forms, needle probes
* ``attend_dense_masked``                -- torch SDPA with a boolean mask
* ``dequantize_fp8``                     -- exact products checked by hand
* ``key_blocks``                         -- column scan of the explicit mask
* ``attend_backward``                    -- torch autograd (float64) through
                                            dense masked attention, central
                                            finite differences, closed forms
                                            (constant values, zero queries,
                                            keys' gradients summing to zero)
* ``linear_key_frames`` / ``linear_mask``  -- complement of the softmax
                                            mask within video pairs, anchors
                                            and window excluded
* ``linear_branch``                      -- pair-by-pair sum over the explicit
                                            mask, closed forms
* ``phi``, ``rms_norm``, ``hybrid_fuse`` -- closed forms, torch routines

No function here is "parity unpinned".
"""

from .local_attn import (  # noqa: F401
    num_frame_blocks,
    window_frames,
    query_blocks,
    key_intervals,
    allowed_mask,
    count_pairs,
    count_pairs_bruteforce,
    attend,
    attend_backward,
    attend_dense_masked,
    key_blocks,
    phi,
    linear_key_frames,
    linear_mask,
    linear_branch,
    rms_norm,
    hybrid_fuse,
    dequantize_fp8,
    sigmoid,
)
