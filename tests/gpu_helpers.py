"""Host <-> device helpers shared by the GPU parity tests (no arithmetic of the method)."""
import numpy as np
import torch

DEV = torch.device("cuda:0")


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16).to(DEV)


def u8_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.uint8)).to(DEV)


def host_u8(t):
    torch.cuda.synchronize()
    return t.view(torch.uint8).cpu().numpy()


def host_bf16_bits(t):
    torch.cuda.synchronize()
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def banner(*a):
    print("[gpu-case]", *a, flush=True)
