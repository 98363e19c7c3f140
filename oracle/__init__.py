"""Oracle: a plain, slow, CPU-only statement of what the expert slot cache computes.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, links or runs
anything here; only the tests, the smoke check and the benchmark's CPU-baseline
leg do.  It shares no code with the HIP library.

* ``oracle.lru`` -- the per-layer slot manager: distinct ids, route rule,
  hits/misses/evictions under the LRU policy and the three alternatives the review
  thread lists (FIFO, LFU, SLRU), map table, remap (vLLM PR "Run MoE models
  exceeding VRAM via expert CPU offloading with GPU cache", section "How it works"
  and the review thread; llama.cpp discussion "Persistent expert slot pool for MoE
  CPU offload", section "Design" and the prefill rule under "Why not the other
  approaches").
* ``oracle.decay`` -- placement by decayed use counts with periodic one-pair moves
  and host reads instead of evictions ("Running 125B MoE on Two 32 GB Cards",
  sections 4.3-4.4).
* ``oracle.router`` -- softmax over the experts, top-k with ties to the lower id,
  gathered gate weights ("Running 125B MoE on Two 32 GB Cards", section 4.2).
* ``oracle.moe`` -- the slot-indexed MoE layer in float64: dequantisation of the
  expert bytes, w13 projection, SwiGLU, w2 projection and the top-k weighted sum.
"""
