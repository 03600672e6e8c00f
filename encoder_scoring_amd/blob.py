"""Writer for the "ESW1" weight blob read by es_load_weights.

Layout (little-endian): a 64-byte header, then the tensors in a fixed order;
matrices and embeddings in the blob's weight dtype (fp32, or bf16 bit
patterns), vectors always fp32.  The C reader in csrc/blob.cpp validates every
size; the layout is documented beside es_load_weights in include/encscore.h.
"""
import struct

import numpy as np

MAGIC = b"ESW1"
VERSION = 1


def tensor_order(n_layers):
    """(name, kind) in blob order; kind "mat" uses the weight dtype, "vec" fp32."""
    out = [("tok_emb", "mat"), ("pos_emb", "mat"), ("norm_g", "vec"), ("norm_b", "vec")]
    for l in range(n_layers):
        p = f"l{l}."
        out += [(p + "w_qkv", "mat"), (p + "b_qkv", "vec"), (p + "w_o", "mat"), (p + "b_o", "vec"),
                (p + "ln1_g", "vec"), (p + "ln1_b", "vec"), (p + "w_1", "mat"), (p + "b_1", "vec"),
                (p + "w_2", "mat"), (p + "b_2", "vec"), (p + "ln2_g", "vec"), (p + "ln2_b", "vec")]
    out += [("head_w", "vec"), ("head_b", "vec")]
    return out


def header(cfg, reward_offset=0.0):
    """64-byte header for a config object with the usual shape attributes."""
    return struct.pack(
        "<4s11I2f2I", MAGIC, VERSION, cfg.n_layers, cfg.hidden, cfg.n_heads, cfg.ffn, cfg.vocab,
        cfg.max_pos, int(cfg.pre_ln), int(cfg.causal), 0, 1 if cfg.bf16 else 0,
        float(cfg.eps), float(reward_offset), 0, 0)


def _expected_shape(cfg, name):
    H, F = cfg.hidden, cfg.ffn
    base = name.split(".")[-1]
    return {"tok_emb": (cfg.vocab, H), "pos_emb": (cfg.max_pos, H), "norm_g": (H,), "norm_b": (H,),
            "w_qkv": (3 * H, H), "b_qkv": (3 * H,), "w_o": (H, H), "b_o": (H,), "ln1_g": (H,),
            "ln1_b": (H,), "w_1": (F, H), "b_1": (F,), "w_2": (H, F), "b_2": (H,), "ln2_g": (H,),
            "ln2_b": (H,), "head_w": (H,), "head_b": (1,)}[base]


def to_bytes(cfg, weights, reward_offset=0.0):
    """Serialise ``weights`` (name -> array) to blob bytes.

    bf16 models: matrices must be uint16 bf16 bit patterns; vectors float32.
    fp32 models: everything float32.
    """
    parts = [header(cfg, reward_offset)]
    for name, kind in tensor_order(cfg.n_layers):
        a = np.asarray(weights[name])
        if tuple(a.shape) != _expected_shape(cfg, name):
            raise ValueError(f"{name}: shape {a.shape}, expected {_expected_shape(cfg, name)}")
        if kind == "mat" and cfg.bf16:
            if a.dtype != np.uint16:
                raise ValueError(f"{name}: bf16 blob needs uint16 bit patterns, got {a.dtype}")
            parts.append(np.ascontiguousarray(a, dtype="<u2").tobytes())
        else:
            if a.dtype != np.float32:
                raise ValueError(f"{name}: expected float32, got {a.dtype}")
            parts.append(np.ascontiguousarray(a, dtype="<f4").tobytes())
    return b"".join(parts)


def write(path, cfg, weights, reward_offset=0.0):
    with open(path, "wb") as f:
        f.write(to_bytes(cfg, weights, reward_offset))
    return path
