"""Helpers shared by the GPU parity tests (host <-> device marshalling only)."""
import numpy as np
import torch

DEV = "cuda:0"


def case(msg):
    """Name the case on stdout before it touches the GPU."""
    print(f"[case] {msg}", flush=True)


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy()).view(torch.bfloat16).to(DEV)


def u8_dev(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8).copy()).to(DEV)


def f32_dev(x):
    return torch.tensor([x], dtype=torch.float32, device=DEV)


def bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def codes(t):
    return t.cpu().numpy()


def f32_bits(x):
    return np.float32(x).view(np.uint32)


def rel_fro(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def same_codes(gpu, ref):
    """e4m3 codes equal bit for bit; a NaN input may come back as either NaN
    code (0x7F or 0xFF), so NaN codes are compared by being NaN."""
    gpu = np.asarray(gpu)
    ref = np.asarray(ref)
    gn = (gpu & 0x7F) == 0x7F
    rn = (ref & 0x7F) == 0x7F
    return bool(((gpu == ref) | (gn & rn)).all())
