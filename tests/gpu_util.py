"""Helpers shared by the GPU parity tests (device transfer of uint32 data as
int32 bits, device synthesis, memory release)."""
import gc
import sys

import numpy as np

TINY_Q = [1073738753, 1073732609]            # N=256: the 2 largest 30-bit primes == 1 mod 512
MED_Q = [536813569, 536690689, 536641537]    # N=4096: the 3 largest 29-bit primes == 1 mod 8192


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def torch_dev():
    import torch

    return torch.device("cuda:0")


def to_dev_u32(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint32).view(np.int32)).to(torch_dev())


def to_dev_i8(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int8)).to(torch_dev())


def to_host_u32(t):
    return t.cpu().numpy().view(np.uint32)


def empty_u32(shape):
    import torch

    return torch.empty(shape, dtype=torch.int32, device=torch_dev())


def empty_bytes(nbytes):
    """A device buffer of nbytes (the relaid DB / hint operands)."""
    import torch

    return torch.empty(nbytes, dtype=torch.uint8, device=torch_dev())


def release():
    import torch

    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
