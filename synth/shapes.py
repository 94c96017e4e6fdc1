"""Parameter-shape lists of the synthetic workloads.

Pure data: lists of (name, shape) in registration order. Nothing here computes
any part of the sharded update; both the CPU oracle side and the GPU side read
these lists to build identical inputs.

Registration order follows each architecture's usual module order (embedding
first, then blocks, then the final norm and head). The flat buffer concatenates
the tensors in exactly this order.
"""
from __future__ import annotations

from math import prod


def numel(shape) -> int:
    return int(prod(shape)) if len(shape) else 1


def tiny():
    """Four 512x512 fp32 tensors, 1,048,576 elements; with N=4 shard r is tensor r."""
    return [(f"w{i}", (512, 512)) for i in range(4)]


def tiny_ragged():
    """Shapes [3,5], [7], [11,13], [1]: 166 elements, so N=4 leaves a tail pad of 2."""
    return [("a", (3, 5)), ("b", (7,)), ("c", (11, 13)), ("d", (1,))]


def gpt2_small():
    """GPT-2 small: token and position embeddings, 12 blocks, final LayerNorm.

    The LM head is tied to the token embedding and so is counted once:
    148 tensors, 124,439,808 elements.
    """
    d, ff, vocab, ctx = 768, 3072, 50257, 1024
    out = [("wte", (vocab, d)), ("wpe", (ctx, d))]
    for i in range(12):
        p = f"h.{i}."
        out += [
            (p + "ln_1.weight", (d,)), (p + "ln_1.bias", (d,)),
            (p + "attn.c_attn.weight", (d, 3 * d)), (p + "attn.c_attn.bias", (3 * d,)),
            (p + "attn.c_proj.weight", (d, d)), (p + "attn.c_proj.bias", (d,)),
            (p + "ln_2.weight", (d,)), (p + "ln_2.bias", (d,)),
            (p + "mlp.c_fc.weight", (d, ff)), (p + "mlp.c_fc.bias", (ff,)),
            (p + "mlp.c_proj.weight", (ff, d)), (p + "mlp.c_proj.bias", (d,)),
        ]
    out += [("ln_f.weight", (d,)), ("ln_f.bias", (d,))]
    return out


def _llama_block(i: int, d: int, kv: int, ff: int):
    p = f"layers.{i}."
    return [
        (p + "self_attn.q_proj.weight", (d, d)),
        (p + "self_attn.k_proj.weight", (kv, d)),
        (p + "self_attn.v_proj.weight", (kv, d)),
        (p + "self_attn.o_proj.weight", (d, d)),
        (p + "mlp.gate_proj.weight", (ff, d)),
        (p + "mlp.up_proj.weight", (ff, d)),
        (p + "mlp.down_proj.weight", (d, ff)),
        (p + "input_layernorm.weight", (d,)),
        (p + "post_attention_layernorm.weight", (d,)),
    ]


def _llama(d: int, kv: int, ff: int, layers: int, vocab: int = 128256):
    out = [("embed_tokens.weight", (vocab, d))]
    for i in range(layers):
        out += _llama_block(i, d, kv, ff)
    out += [("norm.weight", (d,)), ("lm_head.weight", (vocab, d))]
    return out


def llama3_8b():
    """Llama-3-8B: 291 tensors, 8,030,261,248 elements (untied head, final norm)."""
    return _llama(4096, 1024, 14336, 32)


def llama3_8b_block():
    """One Llama-3-8B decoder block (the copy-out unit): 9 tensors, 218,112,000 elements."""
    return _llama_block(0, 4096, 1024, 14336)


def llama_70b():
    """70B Llama shape (hidden 8192, MLP 28672, GQA kv 1024, 80 blocks, vocab 128256).

    723 tensors, 70,553,706,496 elements.
    """
    return _llama(8192, 1024, 28672, 80)


def llama_70b_block():
    """One 70B decoder block: 9 tensors, 855,654,400 elements."""
    return _llama_block(0, 8192, 1024, 28672)


def flat_7p5b():
    """A single flat tensor of 7.5e9 elements."""
    return [("flat", (7_500_000_000,))]


# name -> (shape-list factory, simulated world size N, contribution dtype)
WORKLOADS = {
    "tiny": (tiny, 4, "bf16"),
    "tiny_ragged": (tiny_ragged, 4, "bf16"),
    "gpt2": (gpt2_small, 8, "bf16"),
    "7p5b": (flat_7p5b, 64, "bf16"),
    "llama8b": (llama3_8b, 8, "bf16"),
    "70b": (llama_70b, 64, "f32"),
}


def numels(shape_list):
    return [numel(s) for _, s in shape_list]
