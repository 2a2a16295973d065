"""Synthetic model and workload inputs for the oracle (test infrastructure only).

Weights and inputs come from the shared seeded generator (``inputs``); this
module only arranges them the way the oracle's functions take them.
"""
from __future__ import annotations

import numpy as np

import inputs
from inputs.configs import (BLOCK_NAMES, MOD_SIGMA, NORM_SIGMA, ROW_SIGMA, TEMB_IN, TID_FINAL_SCALE,
                            TID_IMG_IN, TID_MODS, TID_MODS0, TID_MODULATION, TID_NORM_OUT, TID_PREFIX_X,
                            TID_PROJ_OUT, TID_T_LIN1, TID_T_LIN2, TID_TOK, TID_TXT_IN1, TID_TXT_IN2,
                            TID_TXT_NORM, W_SIGMA, block_tid)

from .qi21_oracle import Geometry


class SynthModel:
    """A randomly initialised denoiser of the given ``inputs.ModelSpec``.

    ``block(l)`` regenerates layer l's tensors on demand (a small cache keeps
    the most recent ones), so a 32-layer model never needs all its weights
    in memory at once.
    """

    def __init__(self, spec, cache_layers: int = 2, overrides=None):
        self.spec = spec
        self.layers = spec.layers
        self.geom = Geometry(dim=spec.dim, heads=spec.heads, head_dim=spec.head_dim,
                             inter=spec.inter, in_ch=spec.in_ch, eps=spec.eps,
                             axes=tuple(spec.axes), theta=spec.theta)
        s = spec.seed
        self.img_in = inputs.host_array(s, TID_IMG_IN, (spec.dim, spec.in_ch), W_SIGMA, bf16=spec.bf16)
        self.proj_out = inputs.host_array(s, TID_PROJ_OUT, (spec.in_ch, spec.dim), W_SIGMA, bf16=spec.bf16)
        self.mods0 = inputs.host_array(s, TID_MODS0, (4 * spec.dim,), MOD_SIGMA)
        self._cache = {}
        self._order = []
        self._keep = cache_layers
        self.overrides = overrides or {}

    def time(self) -> dict:
        """The time path's weights ([QI] ``Qi21Dit``: ``t_lin1`` [dim][256],
        ``t_lin2`` [dim][dim], ``modulation`` [4 dim][dim], ``norm_out``
        [dim][dim]; bias-free), drawn like the other matrices."""
        if getattr(self, "_time", None) is None:
            sp, s = self.spec, self.spec.seed
            shapes = {"t_lin1": (TID_T_LIN1, (sp.dim, TEMB_IN)), "t_lin2": (TID_T_LIN2, (sp.dim, sp.dim)),
                      "modulation": (TID_MODULATION, (4 * sp.dim, sp.dim)), "norm_out": (TID_NORM_OUT, (sp.dim, sp.dim))}
            self._time = {k: inputs.host_array(s, tid, shape, W_SIGMA, bf16=sp.bf16) for k, (tid, shape) in shapes.items()}
        return self._time

    def txt(self) -> dict:
        """The txt_in front's weights ([QI] ``Qi21Dit``: ``txt_norm``
        [context_in] (zero-centred: the norm multiplies by w + 1),
        ``txt_in1`` [dim][context_in], ``txt_in2`` [dim][dim]; bias-free);
        context_in = dim here."""
        if getattr(self, "_txt", None) is None:
            sp, s = self.spec, self.spec.seed
            self._txt = {
                "txt_norm": inputs.host_array(s, TID_TXT_NORM, (sp.dim,), NORM_SIGMA),
                "txt_in1": inputs.host_array(s, TID_TXT_IN1, (sp.dim, sp.dim), W_SIGMA, bf16=sp.bf16),
                "txt_in2": inputs.host_array(s, TID_TXT_IN2, (sp.dim, sp.dim), W_SIGMA, bf16=sp.bf16),
            }
        return self._txt

    def block(self, l: int) -> dict:
        if l in self._cache:
            return self._cache[l]
        spec = self.spec
        out = {}
        for j, (name, shape) in enumerate(zip(BLOCK_NAMES, spec.block_shapes())):
            if name.startswith("norm"):
                out[name] = inputs.host_array(spec.seed, block_tid(l, j), shape, NORM_SIGMA, mean=1.0)
            else:
                out[name] = inputs.host_array(spec.seed, block_tid(l, j), shape, W_SIGMA, bf16=spec.bf16)
        out.update(self.overrides.get(l, {}))
        self._cache[l] = out
        self._order.append(l)
        while len(self._order) > self._keep:
            self._cache.pop(self._order.pop(0), None)
        return out


def workload_inputs(w, prefix: int = 0) -> dict:
    """Prefix rows, tokens, modulation and final scale of workload ``w``."""
    spec = w.model
    lp = w.prefix_len(prefix)
    return {
        "x_prefix": inputs.host_array(w.prefix_seed(prefix), TID_PREFIX_X, (lp, spec.dim), ROW_SIGMA),
        "tok": inputs.host_array(w.seed, TID_TOK, (w.n, spec.in_ch), ROW_SIGMA),
        "mods": inputs.host_array(w.seed, TID_MODS, (4 * spec.dim,), MOD_SIGMA),
        "final_scale": inputs.host_array(w.seed, TID_FINAL_SCALE, (spec.dim,), MOD_SIGMA),
    }
