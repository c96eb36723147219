"""Seeded draws generated on the GPU, for workloads too large to draw on the host.

N(0, 1) float32 draws from torch's device generator, rounded to bf16 (round to
nearest even), returned as int16 bit patterns on the device.  Tests copy the
rows they check back to the host for the oracle; those rows are inputs, drawn
here, never values the library computed.
"""


class DeviceDraws:
    def __init__(self, seed, device="cuda"):
        import torch
        self.torch = torch
        self.device = device
        self.gen = torch.Generator(device=device)
        self.gen.manual_seed(seed)

    def bf16(self, shape):
        t = self.torch
        x = t.randn(shape, generator=self.gen, device=self.device, dtype=t.float32)
        return x.to(t.bfloat16).view(t.int16)

    def rms_normalised(self, k_bits, eps=1e-6):
        """Value rows equal to the RMS-normalised key rows (no learned scale),
        computed in float64 from the bf16 keys and rounded to bf16."""
        t = self.torch
        k = k_bits.view(t.bfloat16).double()
        v = k / t.sqrt((k * k).mean(dim=-1, keepdim=True) + eps)
        return v.float().to(t.bfloat16).view(t.int16)
