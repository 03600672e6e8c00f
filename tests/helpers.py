"""Shared test helpers: seeded models on the GPU and oracle comparisons."""
import sys

import numpy as np

from synth.configs import ModelConfig


def say(*a):
    print("[test]", *a, flush=True)
    sys.stdout.flush()


def need_gpu():
    import pytest
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no ROCm GPU visible")
    return torch


def mini(name, pre_ln, causal, bf16, H=64, A=4, F=128, L=2, V=97, P=64, eps=1e-5, seed=7):
    return ModelConfig(name=name, n_layers=L, hidden=H, n_heads=A, ffn=F, vocab=V, max_pos=P,
                       pre_ln=pre_ln, causal=causal, bf16=bf16, eps=eps,
                       seeds={"weights": seed, "requests": seed + 1, "reference": seed + 2})


def bf16_bits_to_f32(t):
    """int16 tensor of bf16 bit patterns -> float32 numpy."""
    a = t.detach().cpu().numpy().view(np.uint16)
    return (a.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(x):
    """float32 numpy -> uint16 bf16 patterns (ties to even), for building test inputs."""
    from synth import round_to_bf16
    return round_to_bf16(np.asarray(x, dtype=np.float32))


def offsets_of(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


def split_decode(bits, M, K):
    """Split-operand layout (es_op_split) -> (hi, lo) uint16 bf16 patterns,
    each [32 ceil(M / 32), K]: element (m, k) half h sits at
    ((((m // 32) (K // 16) + k // 16) 2 + h) 64 + ((k // 8) % 2) 32 + m % 32) 8 + k % 8."""
    M32 = -(-M // 32) * 32
    a = np.asarray(bits).view(np.uint16)[: M32 * K * 2].reshape(M32 // 32, K // 16, 2, 2, 32, 8)
    # [tile][kstep][half][k-octet][row][e] -> [tile][row][kstep][k-octet][e]
    hi = a[:, :, 0].transpose(0, 3, 1, 2, 4).reshape(M32, K)
    lo = a[:, :, 1].transpose(0, 3, 1, 2, 4).reshape(M32, K)
    return hi, lo


def bits_to_f64(bits):
    """uint16 bf16 patterns (numpy) -> float64."""
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
