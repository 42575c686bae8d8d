"""Helpers of the GPU tests: move seeded numpy inputs to the device and back."""
import numpy as np
import torch

from workloads import bf16_bits_to_f32


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> bf16 tensor on cuda:0."""
    return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.bfloat16).to("cuda:0")


def dev_f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda:0")


def host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy float64 (bf16 widened exactly)."""
    t = t.detach().to("cpu")
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f32(t.view(torch.int16).numpy().view(np.uint16)).astype(np.float64)
    return t.numpy().astype(np.float64)


def inputs_to_dev(inp: dict, io: str = "bf16") -> dict:
    out = dict(alpha=dev_f32(inp["alpha"]), beta=dev_f32(inp["beta"]), gates=dev_f32(inp["gates"]))
    for name in ("q", "k", "v"):
        out[name] = dev_bf16(inp[name + "_bits"]) if io == "bf16" else dev_f32(inp[name])
    return out
