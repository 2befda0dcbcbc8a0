"""CPU oracle for the persistent tile-graph megakernel.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import anything here.  The
product path (``tiled_gemm_graph_amd``) never imports, links or calls it,
and this package never imports the product path.  The two share only the
seeded input generator in ``workloads`` (data, no arithmetic).

Contents

``ops``       plain numpy definitions of every op the graphs use (GEMM,
              bias, ReLU, residual, RMSNorm, SiLU-mul, rotary embedding,
              causal grouped-query attention, one-token attention over a KV
              cache with the rotary append), evaluated in fp32 by default.
``graphs``    the workload graphs (the five configurations and the decode
              layer with KV-cache attention) evaluated op by op from the
              same fp16/bf16 input bytes the GPU consumes.
``schedule``  a brute-force re-derivation of the instruction list, tensor
              slots and dependency counters from a graph description and
              per-node tile parameters (MegaKittens Internals, sections
              04-05), used to check the compiler's records exactly.

Parity status of each function is stated in its docstring.  Every numeric
function is pinned in ``tests/test_oracle_*.py`` against brute force,
closed forms or invariants; the rotary embedding's base and pairing are a
reading of the pages (they print no formula) and are marked
"parity unpinned" for those two choices only.
"""
