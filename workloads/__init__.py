"""Seeded synthetic decode workloads shared by the CPU oracle and the HIP path.

This package only draws random numbers and hands out physical block ids (the
role a block manager plays before a kernel runs).  It holds none of the
paged-attention arithmetic: it never computes a slot, an in-block offset, an
address or an attention value.  The oracle (``oracle/``) and the HIP library
each do that on their own from what is produced here.
"""

from .generate import (  # noqa: F401
    Workload,
    POISON_BITS,
    tiny_f32,
    llama3_8b_decode,
    long_context,
    shared_prefix,
    shared_groups,
    mixed_lengths,
    custom,
    normal_values,
    PrefillWorkload,
    prefill,
    llama3_8b_prefill,
)
