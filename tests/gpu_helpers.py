"""Helpers shared by the GPU tests: host <-> device copies of raw bit patterns and a
progress print that names each case before its kernels run."""
import sys

import numpy as np
import torch

DEV = "cuda"


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def bf16_to_dev(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(DEV)


def u8_to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def to_host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def guarded(shape, dtype, pad=4096, fill=0xA5):
    """A tensor view surrounded by canary bytes; returns (view, checker)."""
    elem = torch.empty((), dtype=dtype).element_size()
    n = int(np.prod(shape)) if len(shape) else 1
    padn = pad // elem
    base = torch.empty(n + 2 * padn, dtype=dtype, device=DEV)
    base.view(torch.uint8).fill_(fill)
    view = base[padn: padn + n].view(shape)

    def check():
        raw = base.view(torch.uint8).cpu().numpy()
        head = raw[: padn * elem]
        tail = raw[(padn + n) * elem:]
        return bool((head == fill).all() and (tail == fill).all())

    return view, check
