"""Oracle for the TP-sharded linear step: a plain, slow, CPU reference in float64.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the benchmark's CPU-baseline
leg may import or run anything in this package.  The product path (the HIP library and its
Python binding) never imports it and never falls back to it.

It shares no code with the HIP path: it decodes the storage formats itself, computes with numpy
float64 (a BLAS dgemm is the only library primitive), and lays out buffers with its own loop.

Sources (web pages, cited by title and section):
  [ATLAS-TP]  llm-infra-atlas, "01 · ColumnParallelLinear / RowParallelLinear and the core autograd"
  [ATLAS-BUF] llm-infra-atlas, "05 · grad/param buffer: data structure and read/write loop"
  [MEGA-SRC]  arganzheng.life, "Megatron-LM architecture and source guide"
  [GTP]       NVIDIA Megatron-Core developer guide, "Generalized Tensor Parallelism (GTP)"

Modules:
  numerics  decoding of bf16, E4M3, E8M0 and E2M1 storage formats and NVFP4 blocks (pinned by
            closed-form tables and hand-decoded bytes); the MX quantiser
  linear    fwd / dgrad / fused wgrad-accumulate, brute-force twins for tiny shapes
  layout    the reverse-order, padded grad/param buffer layout
  shapes    parameter counts of the Llama-3.2-1B-shape ledger and its TP=2 shards
"""
from . import numerics, linear, layout, shapes  # noqa: F401
