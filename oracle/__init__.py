"""CPU oracle for the host-memory-centric, layer-streamed training step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link anything under ``oracle/``; only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library: it has its own flat-layout code, its own RoPE table and its
own AdamW, written from the method's description.

Sources (cited by page title and section, see the module docstrings):

* zhichai.net, "MegaTrain：单卡训百亿大模型的突破与实践" (page "zhichai"),
  design points 1-4 of "MegaTrain：以内存为中心的训练新范式".
* blog.travelaiplan.net, "單卡也能練 100B+：MegaTrain 實戰" (page
  "travelaiplan"), "核心功能" 1-3.
* m.lqnn.cn MegaTrain article (page "lqnn"), sections 二 (ParameterState),
  三.1 (double buffering / flat buffers), 三.3 (K-slab pool), 三.4
  (checkpoint recompute), 四 (structure groups).

The pages never write the decoder block down; they call the homogeneous
layers "Llama Transformer layers" (lqnn, 四).  The oracle therefore takes the
plain pre-norm Llama block (RMSNorm, RoPE, causal softmax attention with
grouped KV heads, SwiGLU MLP, untied LM head, mean next-token cross-entropy)
and the AdamW of the optimizer the pages name (lqnn, 二).  Every such reading
is listed with the tests that pin it.

Modules:
  layout   -- flat per-group layout, pack/unpack (lqnn 三.1)
  model    -- block / head / embedding forward and analytic backward, whole-model
              and streamed-with-recompute drivers (zhichai D2, D3; lqnn 三.4)
  moe      -- mixture-of-experts feed-forward, the second structure group (lqnn 四)
  adamw    -- decoupled AdamW on fp32 host state (zhichai D1; lqnn 二)
  accounting -- host-state byte counts (zhichai intro; travelaiplan 核心功能 1)
"""
