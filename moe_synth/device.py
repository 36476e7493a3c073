"""Moves generated inputs to a torch device and lists them as the keyword
arguments of the library binding's make_desc / make_weights (plain dicts:
this module imports neither the binding nor the oracle)."""
from __future__ import annotations

import numpy as np

from .configs import WF_U4, DT_BF16
from .generator import MoeInputs, U4Weights


def _t(a, device, bf16=False, f16=False):
    import torch
    if a is None:
        return None
    if isinstance(a, torch.Tensor):
        return a.to(device)
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).to(device)
        return t.view(torch.bfloat16) if bf16 else (t.view(torch.float16) if f16 else t)
    return torch.from_numpy(a).to(device)


def to_device(inp: MoeInputs, device) -> MoeInputs:
    """Copy a host MoeInputs (numpy) to `device` (torch tensors)."""
    if inp.backend != "numpy":
        return inp
    cfg = inp.cfg
    xb = cfg.act_dtype == DT_BF16
    rb = cfg.router_dtype == DT_BF16
    wb = cfg.weight_format == 1

    def w(m):
        if isinstance(m, U4Weights):
            return U4Weights(_t(m.codes, device), _t(m.scales, device, f16=True),
                             _t(m.mins, device, f16=True), m.K, m.group)
        return _t(m, device, bf16=wb)

    out = MoeInputs(cfg, _t(inp.x, device, bf16=xb), _t(inp.router, device, bf16=rb),
                    _t(inp.router_bias, device), w(inp.gate), w(inp.up), w(inp.down),
                    backend="torch")
    if cfg.shared:
        out.shared_gate_inp = _t(inp.shared_gate_inp, device, bf16=rb)
        out.shared_gate = _t(inp.shared_gate, device, bf16=wb)
        out.shared_up = _t(inp.shared_up, device, bf16=wb)
        out.shared_down = _t(inp.shared_down, device, bf16=wb)
    return out


def desc_kwargs(cfg, normalize_topk=True, gating=0, routed_scale=1.0):
    return dict(hidden=cfg.H, intermediate=cfg.I, num_experts=cfg.E, top_k=cfg.k,
                activation=cfg.act, weight_format=cfg.weight_format, act_dtype=cfg.act_dtype,
                router_dtype=cfg.router_dtype, normalize_topk=normalize_topk,
                shared_intermediate=cfg.Is if cfg.shared else 0, group_size=cfg.group_size,
                gating=gating, routed_scale=routed_scale)


def weights_kwargs(dev: MoeInputs):
    """Keyword arguments for make_weights from a device MoeInputs."""
    kw = dict(router=dev.router, router_bias=dev.router_bias)
    if dev.cfg.weight_format == WF_U4:
        kw["u4"] = {n: (m.codes, m.scales, m.mins)
                    for n, m in (("gate", dev.gate), ("up", dev.up), ("down", dev.down))}
    else:
        kw.update(gate=dev.gate, up=dev.up, down=dev.down)
    if dev.cfg.shared:
        kw.update(shared_gate_inp=dev.shared_gate_inp, shared_gate=dev.shared_gate,
                  shared_up=dev.shared_up, shared_down=dev.shared_down)
    return kw


class HostView:
    """Indexable host view of a device tensor in storage format (uint16 bits
    for bf16/f16), fetching only the slices the oracle asks for."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, idx):
        import torch
        v = self.t[idx]
        if v.dtype in (torch.bfloat16, torch.float16):
            return v.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return v.contiguous().cpu().numpy()


def host_views(dev: MoeInputs) -> MoeInputs:
    """A MoeInputs whose fields read slices back from the device lazily."""
    def hv(m):
        if m is None:
            return None
        if isinstance(m, U4Weights):
            return U4Weights(HostView(m.codes), HostView(m.scales), HostView(m.mins), m.K, m.group)
        return HostView(m)
    out = MoeInputs(dev.cfg, hv(dev.x), hv(dev.router), hv(dev.router_bias), hv(dev.gate),
                    hv(dev.up), hv(dev.down), backend="numpy")
    out.shared_gate_inp = hv(dev.shared_gate_inp)
    out.shared_gate = hv(dev.shared_gate)
    out.shared_up = hv(dev.shared_up)
    out.shared_down = hv(dev.shared_down)
    return out
