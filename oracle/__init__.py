"""Plain, slow fp64 CPU oracle for the tensor-parallel MLP shard, its
sequence-parallel LayerNorm / dropout / residual region, the tensor-parallel
self-attention shard and the vocabulary-parallel cross-entropy head.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP library
never calls it and shares no code with it: no kernels, helpers, tables or
constant generators.  Seeded inputs come from ``tpmlp_inputs`` (which holds no
arithmetic of the method) and are fed to both sides.

Pages cited (by title and section):
  [TUT]   "024｜Megatron-LM：按矩阵结构切分 Transformer，减少模型并行通信"
          (wq-win.github.io/llm/024-megatron.html)
  [SENSE] SenseParrots, 模型并行 (www.xujun.org/note-150970.html)
  [SP]    "Megatron-SP 机制" (t6page.pages.dev, LLM并行通信/序列并行)
  [TRAIN] "Megatron 训练" (lovelonelytime.netlify.app/posts/megatron-learning)
  [EFF]   notes on "Efficient Large-Scale Language Model Training on GPU
          Clusters Using Megatron-LM" (unpurerationalist.github.io)

Every function is written in fp64 NumPy straight from its definition; the
matrix products are ``numpy.matmul`` and nothing is blocked, fused or
reordered beyond what the definition states.

Parity pins (tests/test_oracle_*.py, run with ``-m "not gpu"``):
  * mlp.*        -- finite differences, torch fp64 autograd of the dense
                    layer, sharded == unsharded, t = 1, linearity in G,
                    standard-normal table values, the ReLU counterexample.
  * layernorm.*  -- torch fp64 layer_norm + autograd, projection invariants,
                    finite differences.
  * philox.*     -- Random123 published known-answer vectors.
  * sp_block.*   -- sharded == unsharded (AllReduce = AllGather∘ReduceScatter),
                    finite differences, torch fp64 autograd.
  * vocab_ce.*   -- torch's fp64 cross_entropy and autograd, split == unsplit
                    for every divisor of V, finite differences, the closed
                    form of zero logits.
  * attention.*  -- torch's fp64 scaled_dot_product_attention and autograd,
                    finite differences, heads split over shards == unsplit,
                    uniform attention when the queries are zero, shift
                    invariance of the keys.
No function here is "parity unpinned".
"""

from . import mlp, layernorm, philox, sp_block, attention, vocab_ce  # noqa: F401
