"""Helpers for the GPU tests: move seeded numpy inputs to the device and
bring results back as raw bits.  Not collected by pytest."""
import numpy as np
import torch

import linear_exl3_input_amd as ex
import workloads as wl


def dev16(a: np.ndarray, dtype=torch.int16) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    return t.view(dtype) if dtype != torch.int16 else t


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def weight(t: "wl.Tensors") -> ex.Exl3Weight:
    lay = t.layer
    return ex.Exl3Weight(dev16(t.trellis), dev16(t.suh, torch.float16), dev16(t.svh, torch.float16),
                         lay.bits, lay.codebook, lay.shards)


def x_dev(x_bits: np.ndarray, x_dtype: str = "bf16") -> torch.Tensor:
    return dev16(x_bits, torch.bfloat16 if x_dtype == "bf16" else torch.float16)


def banner(msg: str) -> None:
    print(f"[gpu] {msg}", flush=True)


def rot_layout(x_rot_natural: np.ndarray) -> np.ndarray:
    """The documented x_rot memory order of a natural [S, M, K] array: k-step
    tiles [S, K/32, M, 32], and within a row's 32 values the 4-element chunks
    stored as 0, 2, 1, 3, 4, 6, 5, 7."""
    a = np.asarray(x_rot_natural)
    S, M, K = a.shape
    v = a.reshape(S, M, K // 32, 8, 4)[..., [0, 2, 1, 3, 4, 6, 5, 7], :].reshape(S, M, K // 32, 32)
    return np.ascontiguousarray(v.transpose(0, 2, 1, 3))


def slab_layout(z: np.ndarray) -> np.ndarray:
    """fp32 partials [P, M, N] -> the slab layout [P, ceil(M/4), N, 4]
    (padding rows zero)."""
    P, M, N = z.shape
    M4 = (M + 3) // 4
    pad = np.zeros((P, 4 * M4, N), dtype=z.dtype)
    pad[:, :M] = z
    return np.ascontiguousarray(pad.reshape(P, M4, 4, N).transpose(0, 1, 3, 2))
