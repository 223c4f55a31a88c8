"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no quantization or matmul arithmetic: it only draws random
numbers and rounds them to the storage dtype a workload asks for (by torch's
own dtype conversion). Every draw is numpy PCG64 seeded with
``[workload_id, tensor_id]`` (tensor 0 = weight, 1 = activation,
2 = indices, 3 = the dense layer's bias), so the oracle and the GPU path see
identical bytes.
"""
import numpy as np
import torch

WEIGHT, ACT, INDEX, BIAS = 0, 1, 2, 3


def rng(workload_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([int(workload_id), int(tensor_id)]))


def normal(shape, std, workload_id, tensor_id, dtype="bf16"):
    """N(0, std^2) drawn in fp32, then stored in `dtype`.

    Returns (torch CPU tensor of that dtype, numpy view used by the oracle:
    float32 for f32, uint16 bit patterns for bf16/f16).
    """
    a = rng(workload_id, tensor_id).standard_normal(size=shape, dtype=np.float32)
    a *= np.float32(std)
    return as_dtype(a, dtype)


def as_dtype(a: np.ndarray, dtype: str):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if dtype == "f32":
        return t, t.numpy()
    tt = {"bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    t = t.to(tt)
    return t, t.view(torch.int16).numpy().view(np.uint16)


def topk_distinct(tokens: int, experts: int, k: int, workload_id: int) -> np.ndarray:
    """Per token, k distinct experts drawn uniformly without replacement."""
    keys = rng(workload_id, INDEX).random((tokens, experts))
    return np.argsort(keys, axis=1)[:, :k].astype(np.uint32)


def iota(shape, dtype="f32"):
    """0, 1, 2, ... in row-major order (the pages' Nx.iota examples)."""
    a = np.arange(int(np.prod(shape)), dtype=np.float32).reshape(shape)
    return as_dtype(a, dtype)
