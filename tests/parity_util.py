"""Runs one workload through the HIP library (via the C ABI binding) and the
CPU oracle on the same seeded inputs, and compares them."""
from __future__ import annotations

import json
import os
import sys

import numpy as np

import mixture_experts_ffn_gemv_amd as M
from moe_synth import (generate, norm_weight_values, expert_scale_values, WF_F32, WF_BF16,
                       WF_U4, DT_BF16)
from moe_synth.device import desc_kwargs, weights_kwargs, host_views
from oracle import moe_oracle as O
from oracle.cases import enforce_margin
from oracle_driver import layer_by_expert

TOL = {WF_F32: 1e-4, WF_BF16: 2e-2, WF_U4: 3e-2}
W_TOL = 1e-5


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def rel_err(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.abs(gpu - ref).max() / max(np.abs(ref).max(), 1e-300))


class Case:
    """Device inputs + descriptor + weights for one configuration."""

    def __init__(self, cfg, device="cuda", normalize=True, gating=0, scale=1.0, norm_eps=None,
                 expert_scale=False):
        import torch
        self.cfg = cfg
        self.normalize = normalize
        self.gating = gating
        self.scale = scale
        # per-expert routing scale: the generator's [E] values, or none
        self.expert_scale = expert_scale_values(cfg) if expert_scale else None
        log(f"[case] generate {cfg.name} T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k}")
        self.dev = generate(cfg, backend="torch", device=device)
        self.pre_norm = None
        xform = None
        wkw = weights_kwargs(self.dev)
        if norm_eps is not None:
            nw = norm_weight_values(cfg)
            self.pre_norm = (nw, norm_eps)
            self.norm_weight = torch.from_numpy(nw).to(device)
            wkw["norm_weight"] = self.norm_weight
            xform = lambda X: O.round_to_act(O.rms_norm(X, nw, norm_eps), cfg.act_dtype == DT_BF16)
        if self.expert_scale is not None:
            self.expert_scale_dev = torch.from_numpy(self.expert_scale).to(device)
            wkw["expert_scale"] = self.expert_scale_dev
        self.redraws = enforce_margin(self.dev, xform=xform)
        torch.cuda.synchronize()
        self.desc = M.make_desc(**desc_kwargs(cfg, normalize_topk=normalize, gating=gating,
                                              routed_scale=scale), norm_eps=norm_eps)
        self.weights = M.make_weights(**wkw)
        self.host = host_views(self.dev)

    def forward(self):
        import torch
        log(f"[gpu] moe_ffn_forward {self.cfg.name}")
        out, ids, w = M.moe_ffn_forward(self.desc, self.dev.x, self.weights, return_routing=True)
        torch.cuda.synchronize()
        return out.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()

    def route(self):
        import torch
        log(f"[gpu] moe_route {self.cfg.name}")
        r = M.moe_route(self.desc, self.dev.x, self.weights)
        torch.cuda.synchronize()
        return {k: getattr(r, k).cpu().numpy() for k in ("ids", "weights", "counts", "offsets",
                                                          "perm")}

    # ---------------------------------------------------------------- oracle
    def oracle_routing(self):
        src = O.WeightSource(self.host, cache=False)
        cfg = self.cfg
        X = O.decode_matrix(self.host.x[:], cfg.act_dtype == DT_BF16)
        if self.pre_norm is not None:
            X = O.round_to_act(O.rms_norm(X, *self.pre_norm), cfg.act_dtype == DT_BF16)
        L = O.router_logits(X, src.router(), src.router_bias())
        ids, w = O.route(L, cfg.k, self.normalize, self.gating, self.scale, self.expert_scale)
        return ids, w

    def oracle_outputs(self, tokens, cache=True, residual=None, by_expert=False):
        """The oracle's outputs for `tokens`; by_expert decodes each expert
        once for all of them (bit-identical, for the large shapes)."""
        if by_expert:
            return layer_by_expert(self.host, tokens, normalize=self.normalize,
                                   gating=self.gating, scale=self.scale, pre_norm=self.pre_norm,
                                   residual=residual, expert_scale=self.expert_scale)
        src = O.WeightSource(self.host, cache=cache)
        r = O.moe_ffn(self.host, tokens=tokens, normalize=self.normalize, src=src,
                      gating=self.gating, scale=self.scale, pre_norm=self.pre_norm,
                      residual=residual, expert_scale=self.expert_scale)
        return r["out"]


def record(name, **fields):
    """Append one case's measured errors to the JSON-lines file named by
    MOE_PARITY_LOG (nothing when it is unset)."""
    path = os.environ.get("MOE_PARITY_LOG")
    if not path:
        return
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "a") as f:
        f.write(json.dumps({"case": name, **fields}) + "\n")


def check_case(case: Case, sample_tokens=None, check_route=True, tokens_from_ids=None,
               label=None):
    """Full comparison; returns a dict of the measured errors.
    tokens_from_ids: a function of the oracle's ids giving the tokens to
    compare (instead of sample_tokens)."""
    cfg = case.cfg
    out, ids, w = case.forward()
    ref_ids, ref_w = case.oracle_routing()
    assert (ids == ref_ids).all(), f"routing ids differ at {np.argwhere(ids != ref_ids)[:5]}"
    werr = float(np.abs(w - ref_w).max())
    assert werr <= W_TOL, f"routing weights differ by {werr}"
    res = {"w_err": werr}
    if check_route:
        r = case.route()
        assert (r["ids"] == ref_ids).all()
        assert float(np.abs(r["weights"] - ref_w).max()) <= W_TOL
        cnt, off, perm, _ = O.permutation(ref_ids, cfg.E)
        assert (r["counts"] == cnt).all(), "expert counts differ"
        assert (r["offsets"] == off).all(), "expert offsets differ"
        assert (r["perm"] == perm).all(), "route permutation differs"
    if tokens_from_ids is not None:
        toks = tokens_from_ids(ref_ids)
    else:
        toks = list(range(cfg.T)) if sample_tokens is None else sorted(set(sample_tokens))
    small = cfg.T * cfg.H * cfg.I < (1 << 26)
    ref = case.oracle_outputs(toks, cache=small, by_expert=not small)
    err = rel_err(out[toks], ref)
    # per-token errors too (each token's max |diff| over max |ref| of all sampled tokens)
    tok_err = np.abs(out[toks] - ref).max(axis=1) / max(np.abs(ref).max(), 1e-300)
    log(f"[parity] {cfg.name}: rel err {err:.3e} on {len(toks)} tokens, w err {werr:.2e}")
    record(label or cfg.name, T=cfg.T, tokens=len(toks), out_err=err, w_err=werr,
           tol=TOL[cfg.weight_format], worst_token=int(toks[int(np.argmax(tok_err))]))
    assert err <= TOL[cfg.weight_format], f"{cfg.name}: rel err {err} > {TOL[cfg.weight_format]}"
    assert np.isfinite(out).all()
    res["out_err"] = err
    res["tokens"] = toks
    return res
