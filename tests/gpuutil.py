"""Helpers shared by the GPU parity tests: upload of generated inputs, oracle threads."""
import os

import numpy as np
import torch

import datagen


def oracle_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def to_dev(a: np.ndarray, io: str, dev="cuda") -> torch.Tensor:
    """Upload float32 values as the workload's I/O dtype (bf16 values are exact)."""
    if io == "bf16":
        bits = datagen.bf16_bits(a).view(np.int16)
        return torch.from_numpy(bits).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


def upload_scan(inp: dict, io: str, dev="cuda") -> dict:
    out = {k: to_dev(inp[k], io, dev) for k in ("x", "delta", "B", "C")}
    out["A"] = torch.from_numpy(inp["A"]).to(dev)
    out["Dskip"] = torch.from_numpy(inp["Dskip"]).to(dev)
    return out


def announce(msg: str) -> None:
    print(f"[gpu] {msg}", flush=True)
