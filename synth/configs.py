"""Model shapes and request laws of the five synthetic scoring workloads.

Each workload is named by what it is.  The shapes follow the models the pages
discuss: a compact BERT encoder (SambaNova, "Breakthrough efficiency in NLP
model deployment": TinyBERT for batch-1 online inference), BERT-base-sized
encoders serving variable-length request streams (TurboTransformers review,
"Main results": lengths 2-100 and 5-500), and a GPT-style decoder reward model
with a scalar head on the final token ("Learning to summarize from human
feedback", Compute setup / Method adaptation / Limitations: 1.3B decoder,
summaries under 48 tokens, best-of-N).
"""
from dataclasses import dataclass, field


@dataclass(frozen=True)
class ModelConfig:
    name: str
    n_layers: int
    hidden: int
    n_heads: int
    ffn: int
    vocab: int
    max_pos: int
    pre_ln: bool          # False: post-LN encoder with embedding LN; True: pre-LN + final LN
    causal: bool          # attention mask: False bidirectional within a sequence, True causal
    bf16: bool            # weights stored bf16-exact (activations computed in fp32 by the oracle)
    eps: float            # LayerNorm epsilon
    # request law
    workload: str = ""
    max_tokens: int = 0   # planner budget on |batch| * max_len(batch)
    batch_overhead: int = 1024
    seeds: dict = field(default_factory=dict)

    @property
    def head_dim(self) -> int:
        return self.hidden // self.n_heads


def _seeds(idx: int) -> dict:
    return {"weights": 1000 + idx, "requests": 2000 + idx, "reference": 3000 + idx}


CONFIGS = {
    # 2 layers, hidden 128, 2 heads, FFN 512, vocab 1000, learned positions <= 64,
    # post-LN, fp32; 8 sequences with lengths uniform in 2..32.
    "tiny_fp32": ModelConfig(
        name="tiny_fp32", n_layers=2, hidden=128, n_heads=2, ffn=512, vocab=1000,
        max_pos=64, pre_ln=False, causal=False, bf16=False, eps=1e-12,
        workload="8 sequences, lengths U{2..32}", max_tokens=1024, batch_overhead=0,
        seeds=_seeds(1)),
    # TinyBERT shape: 4 layers, hidden 312, 12 heads of 26, FFN 1200, vocab 30522.
    "tinybert": ModelConfig(
        name="tinybert", n_layers=4, hidden=312, n_heads=12, ffn=1200, vocab=30522,
        max_pos=512, pre_ln=False, causal=False, bf16=True, eps=1e-12,
        workload="fixed lengths 64/128/256 at batch 1 and batch 64", max_tokens=16384,
        seeds=_seeds(2)),
    # BERT-base shape, request stream with lengths uniform in 2..100.
    "bert_base_short": ModelConfig(
        name="bert_base_short", n_layers=12, hidden=768, n_heads=12, ffn=3072,
        vocab=30522, max_pos=512, pre_ln=False, causal=False, bf16=True, eps=1e-12,
        workload="2000 requests, lengths U{2..100}", max_tokens=4096, seeds=_seeds(3)),
    # Same shape, long-tail stream: 1800 x U{5..500} plus 200 x U{400..500}.
    "bert_base_longtail": ModelConfig(
        name="bert_base_longtail", n_layers=12, hidden=768, n_heads=12, ffn=3072,
        vocab=30522, max_pos=512, pre_ln=False, causal=False, bf16=True, eps=1e-12,
        workload="1800 x U{5..500} + 200 x U{400..500}", max_tokens=16384,
        seeds=_seeds(4)),
    # GPT-style decoder reward model, 24 x 2048, 16 heads, FFN 8192, causal, pre-LN;
    # best-of-16 scoring of 64 prompts of 512 tokens, summaries U{8..48}.
    "decoder_rm": ModelConfig(
        name="decoder_rm", n_layers=24, hidden=2048, n_heads=16, ffn=8192, vocab=50257,
        max_pos=1024, pre_ln=True, causal=True, bf16=True, eps=1e-5,
        workload="64 prompts x 16 candidates, prompt 512 + summary U{8..48}",
        max_tokens=16384, seeds=_seeds(5)),
}

ORDERED = ["tiny_fp32", "tinybert", "bert_base_short", "bert_base_longtail", "decoder_rm"]


def get_config(name: str) -> ModelConfig:
    if name not in CONFIGS:
        raise KeyError(f"unknown workload {name!r}; known: {ORDERED}")
    return CONFIGS[name]
