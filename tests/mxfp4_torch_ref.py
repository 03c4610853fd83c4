"""An MXFP4 (transposed banks) expert written independently of the oracle, in torch
float64, for pinning the oracle (not a test module).

Element values come from the literal e2m1 table of the OCP Microscaling spec v1.0
and scales from torch's own e8m0 type (torch.float8_e8m0fnu); the nibble unpacking,
the [K/32, N, 16] block layout, the bias and SiLU are written here from the bank
description alone: blocks hold 32 codes along K per 16 bytes, element 2j in the low
nibble of byte j; one e8m0 scale per 32-element block; a bf16 bias added after each
matmul.
"""
import torch

# OCP MX v1.0 e2m1: sign bit 3, then the 8 magnitudes
E2M1 = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                     -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0], dtype=torch.float64)


def matrix(blocks_u8, scales_u8, n, K):
    """W[n, K] float64 from blocks [K/32, n, 16] u8 and scales [K/32, n] e8m0."""
    b = torch.as_tensor(blocks_u8).reshape(K // 32, n, 16).to(torch.int64)
    codes = torch.stack([b & 0xF, b >> 4], dim=-1).reshape(K // 32, n, 32)
    scale = torch.as_tensor(scales_u8).reshape(K // 32, n).view(torch.float8_e8m0fnu).to(torch.float64)
    vals = E2M1[codes] * scale[:, :, None]                # [K/32, n, 32]
    return vals.permute(1, 0, 2).reshape(n, K)


def bias(u8):
    return torch.as_tensor(u8).view(torch.bfloat16).to(torch.float64)


def expert(rows, H, I):
    """rows: the six bank rows (uint8) in bank order gate_up_blocks, gate_up_scales,
    gate_up_bias, down_blocks, down_scales, down_bias."""
    r = [torch.as_tensor(x).reshape(-1) for x in rows]
    wgu = matrix(r[0], r[1], 2 * I, H)
    wd = matrix(r[3], r[4], H, I)
    return wgu, wd, bias(r[2]), bias(r[5])


def output(x64, rows, H, I):
    """o = Wd (silu(gate) * up) + b_d for activations x64 [m, H] (torch float64)."""
    wgu, wd, bgu, bd = expert(rows, H, I)
    a = x64 @ wgu.T + bgu
    h = torch.nn.functional.silu(a[:, :I]) * a[:, I:]
    return h @ wd.T + bd
