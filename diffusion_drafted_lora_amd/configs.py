"""Model and workload shapes of the Psi-Spec decode step (numbers only, no arithmetic).

The fields mirror ``uno_config`` in ``include/uno.h``.  The five named workloads are:

* ``TINY``     -- 2-layer fp32 decoder (d 64, 4x16 heads, SwiGLU 128, vocab 32 with
                  the last id as MASK), gated LoRA r 8; batch 1, prompt 16, block 4,
                  32 new tokens.  Small enough for the CPU oracle and the
                  losslessness test.
* ``LAYER8B``  -- one Qwen3-8B-shaped layer in bf16 (d 4096, 32 q / 8 kv heads of 128,
                  SwiGLU 12288), LoRA r 128 alpha 256 on all seven projections; KV
                  context 1024; one 16-slot draft forward plus one 16-row verify.
* ``MODEL8B``  -- 36 such layers plus a 151936-column LM head; batch 1, prompt 1024,
                  8192 new tokens, block 16, 16-token KV pages.
* ``MODEL8B_BS128`` -- the same model with 128 concurrent sequences.
* ``DISTILL8B`` -- the same model run as one gated block-causal forward over
                  batch 8 of [x (2048 clean), z1 (2048 MASK)].
"""
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class UnoConfig:
    name: str
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    vocab: int
    lora_rank: int
    lora_alpha: float
    block_size: int
    dtype: str = "bf16"          # "f32" or "bf16" storage
    rope_theta: float = 1.0e6
    rms_eps: float = 1.0e-6
    page_size: int = 16
    qk_norm: bool = False        # Qwen3-style RMSNorm of each q / k head before RoPE
    # workload
    batch: int = 1
    prompt_len: int = 16
    new_tokens: int = 32

    @property
    def mask_id(self) -> int:
        return self.vocab - 1

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def max_len(self) -> int:
        """Positions a sequence may occupy: prompt + new tokens + one block of slack."""
        return self.prompt_len + self.new_tokens + self.block_size + 1

    def with_(self, **kw) -> "UnoConfig":
        return replace(self, **kw)


TINY = UnoConfig(name="tiny-fp32", n_layers=2, d_model=64, n_q_heads=4, n_kv_heads=4,
                 head_dim=16, ffn_dim=128, vocab=32, lora_rank=8, lora_alpha=16.0,
                 block_size=4, dtype="f32", batch=1, prompt_len=16, new_tokens=32)

LAYER8B = UnoConfig(name="qwen3-8b-layer-bf16", n_layers=1, d_model=4096, n_q_heads=32,
                    n_kv_heads=8, head_dim=128, ffn_dim=12288, vocab=151936,
                    lora_rank=128, lora_alpha=256.0, block_size=16, dtype="bf16",
                    batch=1, prompt_len=1024, new_tokens=0)

MODEL8B = LAYER8B.with_(name="qwen3-8b-36L-bf16", n_layers=36, prompt_len=1024,
                        new_tokens=8192)

MODEL8B_BS128 = MODEL8B.with_(name="qwen3-8b-36L-bf16-bs128", batch=128)

DISTILL8B = MODEL8B.with_(name="qwen3-8b-distill-bf16", batch=8, prompt_len=2048,
                          new_tokens=0)

ALL = {c.name: c for c in (TINY, LAYER8B, MODEL8B, MODEL8B_BS128, DISTILL8B)}
