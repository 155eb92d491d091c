"""Seeded synthetic workloads for the paged-attention hot path.

This module only *draws inputs*: context lengths, physical block placement,
slot mappings and N(0, 1) tensors.  It holds none of the method's arithmetic
(no attention, no softmax, no pool logic) and is shared by the tests, the
benchmark and the smoke check; the oracle never imports it and neither does
the library.

The five workloads (the pages benchmark on ShareGPT-sampled lengths with
LLaMA-7B / LLaMA-13B models; no dataset or weights are used here, synthetic
lengths and values of those models' attention shapes stand in for them):

  tiny          4 sequences, L = {1, 17, 33, 100}, 4 heads MHA, D = 64, fp16,
                64-block pool, block tables a seeded permutation of the pool.
  llama7b       64 sequences, 32 heads MHA, D = 128, fp16, L ~ U[128, 2048],
                pool 1.2 x demand, blocks scattered (the headline workload).
  llama13b      128 sequences, 40 heads, D = 128, fp16, L lognormal(median
                400, sigma 1) capped at 2048; groups of 4 share a prompt
                prefix (floor(0.5 * shortest length in the group)).
  llama8b_gqa   256 sequences, 32 query heads over 8 KV heads, D = 128, bf16,
                L ~ U[512, 4096], split partitions of 512 tokens.
  mixed         one step of 8192 tokens at the 8B GQA shape: 4096 decode
                tokens (L ~ U[256, 4096]) + 2 prefill chunks of 2048 query
                tokens over 1024 cached tokens each.
  llama8b_long  32 sequences at the 8B GQA shape, bf16, L ~ U[8192, 32768]:
                contexts longer than one partition's block table (4096
                tokens), library partitioning.

Seeds: workload i (1..5 in the order above) uses seed 4220 + i; llama8b_long
uses 4226.  Host-side
metadata comes from numpy's PCG64; tensors come from a torch.Generator on the
device they are created on.
"""
from __future__ import annotations

from .configs import (  # noqa: F401
    DecodeWorkload, MixedWorkload, SharedWorkload, WORKLOADS,
    make_workload, tiny, llama7b, llama13b_shared, llama8b_gqa, llama8b_long, mixed,
    normal_tensor, torch_dtype,
)
