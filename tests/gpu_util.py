"""Helpers for the GPU tests: device copies of synthetic inputs and a call wrapper."""
import numpy as np
import torch

import verify_matmul_amd as vm

DEV = torch.device("cuda:0")


def dev_u32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).to(DEV)


def dev_u16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


class DevInputs:
    """Device copies of a synth.Inputs."""

    def __init__(self, inp):
        self.inp = inp
        self.qweight = dev_u32(inp.qweight)
        self.scales = dev_u16(inp.scales)
        self.qzeros = None if inp.qzeros is None else dev_u32(inp.qzeros)
        self.act = dev_u16(inp.act)
        self.K, self.N, self.group = inp.K, inp.N, inp.group

    def run(self, M: int, out_dtype=torch.float32, splits=None, waves_k=0, act=None, tile_cols=0) -> np.ndarray:
        a = self.act[:M] if act is None else act
        out = torch.empty((M, self.N), dtype=out_dtype, device=DEV)
        if splits is None and not waves_k and not tile_cols:
            vm.w4a16_gemm(a, self.qweight, self.scales, self.qzeros, self.group, out)
        else:
            vm.w4a16_gemm_ex(a, self.qweight, self.scales, self.qzeros, self.group, out, splits or 0, waves_k,
                             tile_cols)
        torch.cuda.synchronize()
        return out.float().cpu().numpy().astype(np.float64)


def say(*a):
    print(*a, flush=True)
