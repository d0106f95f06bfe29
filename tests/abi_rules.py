"""The broken-geometry cases of the C ABI's validation, each with the words
its error message must use to name the rule (shared by the host tests and
the AddressSanitizer driver; no torch, no library import)."""

SSM_BASE = dict(batch_size=2, sequence_length=8, num_heads=4, num_groups=2, head_dim=16, state_size=32,
                num_rope_angles=8, mimo_rank=1, has_z=True, has_d=True, has_output_norm=False)
SSM_FIELDS = tuple(SSM_BASE)

PRE_BASE = dict(inner_size=64, state_size=16, num_heads=4, num_rope_angles=4, num_groups=1, mimo_rank=1,
                epsilon=1e-5, dt_min=1e-3, dt_max=0.1, a_floor=1e-4)
PRE_FIELDS = tuple(PRE_BASE)

# each broken rule, with the words the error message must use to name it
SISO_BAD = [
    (dict(batch_size=0), "batch_size is 0"), (dict(sequence_length=0), "sequence_length is 0"),
    (dict(num_heads=0), "num_heads is 0"), (dict(num_groups=3), "num_groups 3 does not divide num_heads 4"),
    (dict(head_dim=0), "head_dim is 0"), (dict(head_dim=129), "head_dim 129 is above the limit of 128"),
    (dict(state_size=0), "state_size is 0"), (dict(state_size=129), "state_size 129 is above the limit of 128"),
    (dict(num_rope_angles=65, state_size=128), "num_rope_angles 65 is above the limit of 64"),
    (dict(num_rope_angles=17), "2 * num_rope_angles = 34 state coordinates, but state_size is 32"),
    (dict(mimo_rank=2), "mimo_rank is 2; the single-input scan takes rank 1 only"),
    (dict(has_output_norm=True), "has_output_norm is set"),
    (dict(num_heads=4, num_groups=8), "num_groups 8 does not divide num_heads 4"),
]

MIMO_BAD = [(dict(mimo_rank=0), "mimo_rank 0 is outside 1..8"), (dict(mimo_rank=9), "mimo_rank 9 is outside 1..8"),
            (dict(head_dim=129), "head_dim 129 is above"), (dict(num_groups=3), "does not divide"),
            (dict(num_rope_angles=17), "2 * num_rope_angles = 34"), (dict(has_output_norm=2), "flag has_output_norm is 2")]

PRE_BAD = [(dict(inner_size=0), "inner_size is 0"), (dict(state_size=0), "state_size is 0"),
           (dict(num_heads=0), "num_heads is 0"), (dict(num_groups=0), "num_groups is 0"),
           (dict(mimo_rank=0), "mimo_rank is 0"), (dict(num_rope_angles=9), "2 * num_rope_angles = 18"),
           (dict(epsilon=0.0), "epsilon is 0; it must be above zero"),
           (dict(epsilon=float("nan")), "epsilon is not a finite number"),
           (dict(dt_min=0.0), "dt_min is 0; it must be above zero"), (dict(dt_min=0.2), "dt_min 0.2 is above dt_max 0.1"),
           (dict(dt_max=float("inf")), "dt_max is not a finite number"),
           (dict(a_floor=0.0), "a_floor is 0; it must be above zero"), (dict(a_floor=-1.0), "a_floor is -1")]
