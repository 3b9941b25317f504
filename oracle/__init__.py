"""Plain fp64 CPU oracle for packed-sequence causal attention with EOD reset.

TEST INFRASTRUCTURE ONLY. Only the test suite, the package's smoke check and
the benchmark's CPU-baseline leg may import this package. The product path
(the C-ABI library and its Python binding) never imports, calls or links it,
and this package imports nothing from the product path.

What it computes, and where that is stated ("kvallgather cp thd load balance",
Ascend/MindSpeed pull request, sections "What this PR does / why we need it?"
and "Does this PR introduce any user-facing change?"):

* load-balanced KV-all-gather context parallelism for THD-packed input: each
  rank keeps a shard of the queries, K and V are all-gathered in rank order;
* EOD-aware symmetric partitioning: every packed subsequence (document) is cut
  into 2*cp equal chunks and rank r owns chunks r and 2*cp-1-r;
* every subsequence length must be divisible by 2*cp;
* causal attention with the attention mask reset at every EOD, i.e. a query
  attends to the keys of its own document at or before its own position;
* MHA, GQA and expanded-MLA head shapes.

Modules:
  partition  the per-rank query map, the rank-major K/V row map, chunk offsets
  metadata   the per-tile document/causal bounds the GPU path consumes
             (an interface contract; parity unpinned beyond its definition)
  attention  fp64 forward (O, LSE) and backward (dQ, dK, dV), plus a pure
             Python loop version for tiny inputs

Parity status: every function here is pinned by the CPU tests
(tests/test_oracle_*.py) except the tile work order of metadata.order, which
has no truth outside its own definition ("parity unpinned").
"""
