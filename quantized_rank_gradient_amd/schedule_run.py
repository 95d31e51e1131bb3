"""Driver of the layer-adaptive refresh schedule over a drifting-subspace workload.

The schedule itself (AIMech curated page on Q-GaLore, mechanism claim "layer-adaptive
subspace cosine schedule", paper Section 3.1): each layer refreshes its projection from the
gradient at an interval; at every refresh after the first, the new projection is compared
with the previous one and a similarity above gamma doubles that layer's interval.

This module is caller-side code around the library: it generates the drifting gradients
(workloads.drift_gradient_device) and, for each due layer, the Gaussian sketch of the
refresh; the library computes the new INT4 projection (qgalore_refresh_proj: randomized range
finder with two power iterations), the batched similarity test, the schedule bookkeeping and
the grouped optimizer step of every layer at every step. refresh="torch" computes the new
projection with the same algorithm in torch instead (comparison).
"""
from __future__ import annotations

import time

import torch

from . import binding as B
from . import workloads as WL


class ScheduleRun:
    def __init__(self, cfg: WL.Config, device: str = "cuda", delta0: int = WL.SCHEDULE_DELTA0,
                 gamma: float = WL.SCHEDULE_GAMMA, debug_layers=(), refresh: str = "library",
                 oversample: int = 8, power_iters: int = 2):
        """debug_layers: indices of layers whose R and U the step also writes out (R_out,
        U_out), for checking. refresh: "library" or "torch" (see the module docstring)."""
        if refresh not in ("library", "torch"):
            raise ValueError(f"unknown refresh {refresh!r}")
        self.refresh, self.oversample, self.power_iters = refresh, oversample, power_iters
        self.cfg, self.r = cfg, cfg.r
        dev = torch.device(device)
        self.basis, self.rho, self.G, self.layers = [], [], [], []
        for k, L in enumerate(cfg.layers):
            self.basis.append(WL.drift_basis_device(cfg, L, device=dev))
            self.rho.append(WL.drift_rate(cfg, k))
            G = torch.empty((L.m, L.n), dtype=torch.bfloat16, device=dev)
            self.G.append(G)
            ng = B.n_groups(self.r * L.n)
            self.layers.append(B.LayerTensors(
                L.layer_id, G, WL.weights_int8_device(cfg, L, device=dev),
                torch.full((B.n_groups(L.m * L.n),), cfg.w_scale, device=dev),
                torch.zeros(((L.m * self.r + 1) // 2,), dtype=torch.uint8, device=dev),
                torch.zeros((B.n_groups(L.m * self.r),), dtype=torch.float32, device=dev),
                torch.zeros((self.r, L.n), dtype=torch.int8, device=dev),
                torch.zeros(ng, device=dev),
                torch.zeros((self.r, L.n), dtype=torch.int8, device=dev),
                torch.zeros(ng, device=dev), self.r))
        self.R_out = [torch.empty((self.r, L.n), device=dev) if k in debug_layers else None
                      for k, L in enumerate(cfg.layers)]
        self.U_out = [torch.empty((L.m, L.n), device=dev) if k in debug_layers else None
                      for k, L in enumerate(cfg.layers)]
        self.plan = B.Plan(self.layers, hp=dict(lr=cfg.lr, beta1=cfg.beta1, beta2=cfg.beta2,
                                                eps=cfg.eps, alpha=cfg.alpha),
                           R_out=self.R_out, U_out=self.U_out)
        # with the separate dequant pass (INT4 ranks the MFMA kernels cannot dequantize
        # themselves), dequantized projections are kept between steps and a refresh marks its
        # layer changed; inline-dequantized layers keep nothing
        self.plan.cache_proj(True)
        self.ws = B.alloc_workspace(self.plan.workspace_bytes)
        self.cws = B.alloc_workspace(B.cossim_batch_workspace_bytes(self.r, 32))
        self.rws = None
        if refresh == "library":
            self.rws = B.alloc_workspace(max(
                B.refresh_workspace_bytes(L.m, L.n, self.r, oversample) for L in cfg.layers))
        self.cs_out = torch.zeros(len(self.layers), dtype=torch.float32, device=dev)
        self.sched = [B.Schedule(delta0, gamma) for _ in self.layers]
        self.refreshed_at = [None] * len(self.layers)   # step of each layer's current P
        self.delta0, self.gamma = delta0, gamma
        self.times = dict(gradients=0.0, subspaces=0.0, similarity=0.0, step=0.0)
        self.tests = 0

    def _timed(self, key, fn):
        torch.cuda.synchronize()
        t0 = time.time()
        out = fn()
        torch.cuda.synchronize()
        self.times[key] += time.time() - t0
        return out

    def step(self, t: int, on_test=None, before_step=None, after_step=None):
        """Step t (0-based): gradients G_t, due refreshes with their similarity tests, then the
        grouped optimizer step (library step number t + 1). Hooks: on_test(layer, t, CosSim,
        (P_q, P_s) new, (P_q, P_s) old, step of the old projection); before_step(t) and
        after_step(t) around the optimizer step."""
        cfg = self.cfg

        def gradients():
            for k, L in enumerate(cfg.layers):
                WL.drift_gradient_device(cfg, L, self.basis[k], self.rho[k], t, out=self.G[k])
        self._timed("gradients", gradients)

        due = [k for k, s in enumerate(self.sched) if s.due(t)]
        if due:
            def subspaces():
                out = {}
                for k in due:
                    L = cfg.layers[k]
                    if self.refresh == "torch":
                        P = WL.top_subspace_device(cfg, L, self.G[k], self.r, t,
                                                   self.oversample, self.power_iters)
                        out[k] = B.quantize_proj(P)
                    else:
                        Om = WL.sketch_device(cfg, L, self.r + self.oversample, t,
                                              device=self.G[k].device)
                        out[k] = B.refresh_proj(self.G[k], self.r, Om, self.power_iters,
                                                workspace=self.rws)
                return out
            new = self._timed("subspaces", subspaces)
            tested = [k for k in due if self.sched[k].count > 0]
            vals = {}
            if tested:
                pairs = [(*new[k], self.layers[k].Pq, self.layers[k].Ps, cfg.layers[k].m)
                         for k in tested]
                self._timed("similarity", lambda: B.cossim_batch(pairs, self.r, self.cs_out,
                                                                 workspace=self.cws))
                vals = dict(zip(tested, self.cs_out[: len(tested)].cpu().tolist()))
                self.tests += len(tested)
            for k in due:
                if on_test is not None and k in vals:
                    on_test(k, t, vals[k], new[k], (self.layers[k].Pq, self.layers[k].Ps),
                            self.refreshed_at[k])
                self.sched[k].refresh(t, vals.get(k))
                self.refreshed_at[k] = t
                self.layers[k].Pq.copy_(new[k][0])
                self.layers[k].Ps.copy_(new[k][1])
                self.plan.proj_changed(k)
        if before_step is not None:
            before_step(t)
        self._timed("step", lambda: self.plan.step(t + 1, WL.SR_SEED, self.ws))
        if after_step is not None:
            after_step(t)

    def run(self, steps: int | None = None, **hooks):
        for t in range(self.cfg.steps if steps is None else steps):
            self.step(t, **hooks)
        return self.summary()

    def summary(self) -> dict:
        counts = [s.count for s in self.sched]
        fixed = len(range(0, self.cfg.steps, self.delta0))
        total_fixed = fixed * len(counts)
        return dict(refresh=self.refresh,
                    svds=int(sum(counts)), svds_fixed_interval=int(total_fixed),
                    svds_saved=round(1.0 - sum(counts) / total_fixed, 4),
                    similarity_tests=self.tests,
                    per_layer_counts=counts,
                    seconds={k: round(v, 2) for k, v in self.times.items()})

    def close(self):
        self.plan.close()
