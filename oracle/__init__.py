"""CPU oracle for decode attention over a KV cache — TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this package. The
library's product path never calls it, and it shares no code, table or helper with the HIP path.

Everything here is plain and slow on purpose: NumPy in float64 (inputs stored as fp32, fp16 or
fp8-e4m3 are widened exactly), pure-Python bookkeeping for the block pool, and no blocking, fusion
or reordering beyond what the definitions state.

Pages cited (titles as printed; section numbers are the pages' own):
  * "LLM Inference Acceleration -- KV Cache" (大模型推理加速——KV Cache篇)
  * "KV Cache Mechanism Explained" (KV缓存机制解析：优化大型语言模型推理性能)
  * "From Neuron to GPT -- KV cache chapter" (键值缓存)
  * "KV Cache and PagedAttention" (KV Cache与PagedAttention：大模型推理显存优化方案)

Modules:
  attention  -- softmax(q.K^T*scale).V: definition, full causal recompute, naive cached path
  codecs     -- fp16 and OCP fp8-e4m3 codecs; the per-block running-amax fp8 write rule
  pool       -- PoolModel: block pool with first-fit, refcounts, fork and copy-on-write
  caches     -- contiguous and paged cache storage models, gather, and decode through them
  accounting -- KV-cache byte and block-count formulas

Parity status: every function is pinned by a -m "not gpu" test against a value the pages print,
a closed form, an independent high-precision evaluation, or brute force; see tests/test_oracle_*.
"""
