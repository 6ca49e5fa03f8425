"""CPU reference ("oracle") for the spatially pipelined MoE decode layer.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check of the entry module
and the benchmark's CPU-baseline leg may import this package; the product path
(the HIP library and its Python binding) never does, and shares no code with it.

Plain, slow, obviously correct float64 numpy. Every function cites the passage
it follows in "SubGPU Pipelining: Intra-GPU Fine-Grained Spatial Parallelism
for LLM Inference" (Andoorveedu et al., arXiv:2611.14904): the operators of one
MoE transformer layer listed in its Figure 3, the execution model of its
section 3 (equations 1-6), the search-space count of section 3.3 (equation 7)
and the allocation refinement of section 4.2 (Algorithm 2). Where the pages
leave a step open, the reading taken is stated in the function's docstring.

Modules:
  layer     - the decode layer: RMSNorm, QKV projection, KV append, GQA decode
              attention with sinks (full and sliding window), output
              projection + residual, router top-k, token->expert permutation,
              SwiGLU experts, weighted combine + residual; whole iterations.
  numerics  - bf16 and OCP E4M3 rounding / decoding.
  schedule  - the augmented task DAG, the max-plus makespan, configuration
              counts and pairwise-line allocation refinement.
"""
