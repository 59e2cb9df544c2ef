"""Device-side seeded inputs (torch) for the full-size workloads.

Weights of the Llama-shaped stacks (15 GB and 29.5 GB of bf16) are drawn on
the GPU with torch's seeded Philox generator, so they never cross PCIe; tests
copy the rows they check back to the host. Holds none of the verification
method's arithmetic.
"""

import numpy as np
import torch


def generator(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & 0x7FFFFFFFFFFFFFFF)
    return g


def normal_bf16(shape, std, seed, device="cuda"):
    """bf16 tensor of N(0, std^2) draws (fp32 normals rounded to nearest even)."""
    z = torch.randn(shape, generator=generator(seed, device), device=device, dtype=torch.float32)
    if std != 1.0:
        z.mul_(std)
    out = z.to(torch.bfloat16)
    del z
    return out


def e4m3_normal_codes(shape, std, seed, device="cuda"):
    """uint8 FP8 E4M3 codes of N(0, std^2) draws clamped to [-448, 448]."""
    z = torch.randn(shape, generator=generator(seed, device), device=device, dtype=torch.float32)
    if std != 1.0:
        z.mul_(std)
    z.clamp_(-448.0, 448.0)
    out = z.to(torch.float8_e4m3fn).view(torch.uint8)
    del z
    return out


def w8_row_scales(d_out, base, seed, device="cuda"):
    """float32 [d_out]: base * (0.75 + 0.5 u), u uniform."""
    u = torch.rand((d_out,), generator=generator(seed, device), device=device, dtype=torch.float32)
    return (u.mul_(0.5).add_(0.75)).mul_(base)


def normal_f32(shape, std, seed, device="cuda"):
    z = torch.randn(shape, generator=generator(seed, device), device=device, dtype=torch.float32)
    if std != 1.0:
        z.mul_(std)
    return z


def uniform_f32(shape, seed, device="cuda"):
    return torch.rand(shape, generator=generator(seed, device), device=device, dtype=torch.float32)


def gumbel_max_tokens(draft_logits, seed):
    """Drafter stand-in on the device: one draw per row of softmax(draft
    logits) by the Gumbel-max trick; [B][K][V] fp32 -> int32 [B][K]."""
    u = torch.rand(draft_logits.shape, generator=generator(seed, draft_logits.device),
                   device=draft_logits.device, dtype=torch.float64)
    g = -torch.log(-torch.log(u))
    return torch.argmax(draft_logits.double() + g, dim=-1).to(torch.int32)


def from_bits(bits, device="cuda"):
    """uint16 bf16 bit patterns (numpy) -> bf16 device tensor."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(device)


def to_bits(t):
    """bf16 tensor -> uint16 bit patterns (numpy, host)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
