"""Small helpers for the GPU parity tests: move uint16 bit arrays between the
host (numpy, as the oracle uses them) and the device (torch), bit for bit."""

import numpy as np
import torch


def dev_bf16(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def dev_f16(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.float16).cuda()


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def host_bits(t):
    """Any 16-bit device tensor -> numpy uint16 bit patterns."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_u8(t):
    return t.detach().contiguous().cpu().numpy()


def host_f32(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.detach().cpu().numpy().astype(np.float64)


def report(name, **kv):
    print(f"[{name}] " + " ".join(f"{k}={v}" for k, v in kv.items()), flush=True)
