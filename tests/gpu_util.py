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
