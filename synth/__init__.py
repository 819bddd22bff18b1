"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

This package draws random numbers and lays out chunk tables; it holds none of
the method's arithmetic (no rotation, no attention).  Everything here is plain
numpy so that the oracle and the GPU tests consume byte-identical inputs.
"""
from .workloads import (  # noqa: F401
    CHUNK_DTYPE,
    FRESH,
    ROW,
    D_LATENT,
    D_ROPE,
    Workload,
    bf16_bits_from_f32,
    randn_bf16,
    make_workload,
    WORKLOADS,
    random_table,
    tiny_decode,
    rotate_gather_batch,
    rotate_gather_cdc_batch,
    batched_decode,
    long_decode,
    tail_prefill,
    token_requests,
    nonabsorbed_inputs,
    manifest,
)
