"""CPU oracle for the Psi-Spec draft-and-verify decode step of diffusion-augmented LLMs (Uno).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call, link or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (``diffusion_drafted_lora_amd``) and imports nothing from it; the two meet
only at the seeded inputs that the tests hand to both.

The oracle is a plain, slow reading of the method in float64 numpy (with an
optional bfloat16 rounding at the storage points the library uses, so that bf16
configurations can be compared), written for a reader to check against the pages.

Citations name the web page and its section.  The pages are:

* [summary]  "Unlocking Lossless Speedups in LLMs via Discrete Diffusion", the
  ai-papers-daily Chinese summary; sections "方法关键点" (method key points) and
  "关键实验" (key experiments).
* [abstract] the shd-paper.top listing of the same paper, section "摘要（原文）"
  (the original abstract).
* [blog]     the shibing624 reading notes "不砸掉重来，给自回归 LLM 装一对'扩散翅膀'：
  Uno 的无损加速之路"; sections "方法核心：一个模型，两套权重" (method core: one
  model, two weight sets), "Diffusion Distillation：一步蒸馏 + 块级扩散" (one-step,
  block-wise distillation), "Ψ-Spec 采样器：起草、验证、两种模式" (the Psi-Spec
  sampler: draft, verify, two modes), "我的判断" (the author's assessment).

Modules:
  rng      Philox4x64-10, the 24-bit uniform, the integer inverse-CDF sampler.
  model    the decoder forward with gated LoRA, RoPE, GQA and a KV cache.
  psispec  prefill, draft, verify, accept/resample, commit, generation loop (top-p optional).
  distill  the [x, z1] block-causal forward with teacher/student logits and TV.
  nucleus  the top-p truncation of a probability row (exact fixed-point reading).
  distill_grad  the block-wise TV loss and its gradient with respect to the LoRA
           (base frozen), layer by layer over the z1 rows.
  tree     the tree sampler: K drafted chains, one verify per chain, recursive
           rejection along the tree of common prefixes.
"""
