"""CPU oracle for attention over a paged KV cache — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct implementation of what the paged-KV path
computes, written from the pages that describe the method:

* "Project 17: Production Serving: Continuous Batching and PagedAttention"
  (llm-under-the-hood), sections "The Concept", "Step 4: Implement the paged
  KV cache" and "Step 6: Implement attention over paged storage";
* "Continuous Batching" (infra.pidoku inference-engineering notes), sections
  "4. Tiny example", "5. Technical explanation" and "6. Under the hood";
* "Build a pure-Python continuous batching LLM serving engine from scratch"
  (martinuke0), "Step 2: Implement the PagedAttention KV Cache Manager";
* the tiny-vllm code reading, part 7 (jaehun.me), "Uploading the active arrays
  to the GPU" and "Termination and returning blocks".

Floating point is float64 on exactly decoded inputs; integer work (free lists,
block tables, slot mappings, the scheduler step) is executed step by step.

Only tests/, the smoke check in __graft_entry__ and the CPU-baseline leg of
bench.py may import or call anything in this package. It shares no code with
the HIP library and imports nothing from it.

Parity status of each part is stated in the module that implements it; the
scheduler step (scheduler.py) is pinned by invariants only (parity unpinned
beyond them: the pages print no worked trace).
"""

from . import allocator, metadata, fp8, cache, attention  # noqa: F401
