"""fp64 CPU oracle for the halo-sharded conv + GroupNorm layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only the tests, the smoke check and the benchmark's CPU-baseline leg may
import, call or execute it.  It shares no code with the HIP library or its
Python binding; the only code both sides use is the seeded input module
`synth`, which holds no arithmetic of the method.

Every function is pinned by CPU tests (brute force on tiny volumes, delta
kernels, linearity, torch fp64 as an independent library, GroupNorm closed
forms, sharded == unsharded; the input gradient by the adjoint identity,
brute force and torch's fp64 autograd; the weight gradient by the adjoint
identity in the weights, brute force and torch's fp64 autograd; the GroupNorm backward by torch's
fp64 autograd and central finite differences; pooling and the strided conv by
brute force, torch's fp64 ops, and the sharded form; the transposed conv by
the adjoint identity with the strided conv, brute force and torch's fp64
conv_transpose; `widen` for bf16 by torch's own bfloat16 -> float64
conversion over every finite bit pattern, and for fp32 by the exact round
trip).
"""
from .reference import (  # noqa: F401
    widen, zero_pad, conv_valid, conv_same, conv_same_dgrad, conv_same_wgrad, conv_same_slabbed, conv_at,
    group_moments, group_norm, group_norm_apply, group_norm_backward, group_sums_onepass,
    pool_valid, pooled_shard_sizes, pool_bruteforce, conv_strided, strided_shard_sizes,
    conv_strided_bruteforce, conv_transposed, conv_transposed_bruteforce,
    shard_offsets, shard_grid, padded_shard, halo_message, halo_directions,
    sharded_forward, conv_bruteforce, conv_dgrad_bruteforce, conv_wgrad_bruteforce,
    group_norm_bruteforce,
)
