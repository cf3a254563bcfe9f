"""Place a workload's seeded inputs in device memory (torch tensors on cuda).

The routed MXFP4 bank (about 21 GB at the full layer shape) is written in place
by the device fill kernels; everything else is generated on the host and
copied.  Holds none of the layer's arithmetic.
"""
from dataclasses import dataclass, field

import numpy as np
import torch

from . import (fill_routed_bank_device, fill_rvq_bank_device, routed_bank, routed_sizes, router,
               rvq_codebooks, rvq_expert, rvq_sizes, shared_bank, x as gen_x)
from .configs import LayerConfig


def _to_dev_bf16(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)


def activations(cfg: LayerConfig, device="cuda", t0: int = 0, t1: int = None) -> torch.Tensor:
    a = gen_x(cfg, t0, t1)
    if cfg.x_dtype == "f32":
        return torch.from_numpy(a).to(device)
    return _to_dev_bf16(a, device)


@dataclass
class DeviceWorkload:
    cfg: LayerConfig
    x: torch.Tensor
    w_router: torch.Tensor
    routed: dict            # name -> uint8 tensor [E][rows][bytes]
    shared: dict            # name -> bf16 tensor (empty when n_shared == 0)
    extra: dict = field(default_factory=dict)


def build(cfg: LayerConfig, device="cuda", routed_on_device: bool = None) -> DeviceWorkload:
    if routed_on_device is None:
        routed_on_device = cfg.E * cfg.d * cfg.f > (1 << 24)
    x = activations(cfg, device)
    wr = _to_dev_bf16(router(cfg), device)
    sz = routed_sizes(cfg)
    shapes = dict(w13=(cfg.E, 2 * cfg.f, cfg.d // 2), w13_scale=(cfg.E, 2 * cfg.f, cfg.d // 32),
                  w2=(cfg.E, cfg.d, cfg.f // 2), w2_scale=(cfg.E, cfg.d, cfg.f // 32))
    if routed_on_device:
        routed = {k: torch.empty(shapes[k], dtype=torch.uint8, device=device) for k in sz}
        fill_routed_bank_device(cfg, {k: v.data_ptr() for k, v in routed.items()},
                                torch.cuda.current_stream().cuda_stream)
    else:
        host = routed_bank(cfg)
        routed = {k: torch.from_numpy(host[k]).to(device) for k in sz}
    shared = {}
    if cfg.n_shared > 0:
        sh = shared_bank(cfg)
        shared = {k: _to_dev_bf16(v, device) for k, v in sh.items()}
    return DeviceWorkload(cfg, x, wr, routed, shared)


def build_rvq(cfg: LayerConfig, device="cuda", on_device: bool = None) -> dict:
    """The RVQ3 routed bank of cfg in device memory: w13 [E][3][d/128][2f][16],
    w2 [E][3][f/128][d][16] uint8 indices (device fill, or host for small
    banks) and their fp32 codebooks w13_cb, w2_cb [E][3][256][8]."""
    if on_device is None:
        on_device = cfg.E * cfg.d * cfg.f > (1 << 24)
    shapes = dict(w13=(cfg.E, 3, cfg.d // 128, 2 * cfg.f, 16), w2=(cfg.E, 3, cfg.f // 128, cfg.d, 16))
    if on_device:
        bank = {k: torch.empty(v, dtype=torch.uint8, device=device) for k, v in shapes.items()}
        fill_rvq_bank_device(cfg, {k: v.data_ptr() for k, v in bank.items()},
                             torch.cuda.current_stream().cuda_stream)
    else:
        ex = [rvq_expert(cfg, e) for e in range(cfg.E)]
        bank = {k: torch.from_numpy(np.stack([x[k] for x in ex])).to(device) for k in shapes}
    for k in ("w13", "w2"):
        bank[k + "_cb"] = torch.from_numpy(rvq_codebooks(cfg, 0, cfg.E, k)).to(device)
    return bank
