"""Plain, slow, float64 CPU oracle of the HySparse2 Cross-Decoder hybrid-block path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library or its Python binding, and it imports nothing from either.

Sources (five web write-ups of one announcement; cited by site, page title and
section, never by a line of any copy of them):

* ithome page -- IT之家 "小米公开 MiMo-V3 核心架构 HySparse2：面向长程多轮 Agent
  优化推理效率" (the most direct copy of the team's own text).  Its sections:
  the KV-sharing overview, "KV Reuse：在同一 Hybrid Block 内，复用 KV 与选择结果",
  the token-level selection and recent-window paragraphs that follow it, and
  the prefill early-exit paragraphs.
* cnyes page -- 量子位 repost "MiMo-V2.6剛發佈，羅福莉就開始劇透MiMo-V3了",
  sections "預填充只走前半程" and "檢索精確到token".
* toolnavs page -- "Xiaomi stellt HySparse2 vor" (Japanese), sections
  "HySparse2 がやったこと" and "Prefill は半分で終わる".
* ai-bio page -- "小米 MiMo-V3 – 小米 MiMo 团队公布的下一代长上下文基础模型",
  sections "两级 KV 共享：KV 桥接与 KV 重用" and "token 级稀疏与近期 Token 强制窗口".
* dpshk page -- news item on HySparse2, sections "02 / ...预填充只跑前半段" and
  "03 / 从按“块”找线索，改成按单个Token找".

What the pages fix, restated: a hybrid block is one full-attention layer
followed by several sparse-attention layers; the full layer picks important
positions from its own attention scores; the sparse layers reuse that layer's
KV cache and its selection indices; selection is per token, always includes
the 128 most recent tokens and adds 1024 global tokens taken from outside that
window; each Cross-Decoder full layer projects its own K and V from the input
hidden state of the matching Self-Decoder full layer, with its own
projections; the cache is stored in FP8.

Readings where the pages are silent (score definition, tie rule, FP8 format,
scale granularity, masking, ...) are listed with each function.

Modules:
  bf16       -- bfloat16 storage decode / round-to-nearest-even encode
  e4m3       -- OCP E4M3FN codec written from the format definition
  attention  -- full attention, selection scores, sparse attention
  selection  -- top-k global + recent-window selection
  bridge     -- KV Bridging projection and its FP8 / bf16 storage
  block      -- one hybrid block: full layer + select + sparse layers
"""

from . import bf16, e4m3, attention, selection, bridge, block  # noqa: F401
