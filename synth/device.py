"""Seeded device-side random inputs for the bench (input generation only).

Large workloads (hundreds of MB of cached K/V) are generated on the GPU with a
seeded torch generator instead of numpy, so the bench sets up in seconds.
"""

from __future__ import annotations

import torch


class DeviceRandom:
    def __init__(self, seed: int, device="cuda"):
        self.g = torch.Generator(device=device)
        self.g.manual_seed(seed)
        self.device = device

    def bf16(self, shape, mean: float = 0.0, std: float = 1.0) -> torch.Tensor:
        """N(mean, std) rounded to bf16 (round to nearest even)."""
        x = torch.randn(shape, generator=self.g, device=self.device, dtype=torch.float32)
        if std != 1.0 or mean != 0.0:
            x = x * std + mean
        return x.to(torch.bfloat16)
