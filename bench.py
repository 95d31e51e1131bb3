"""Benchmark of the Q-GaLore optimizer step on one MI355X.

A step is one pass of the whole hot path over a LLaMA-7B-shaped layer set (32 blocks x
{q, k, v, o 4096x4096; gate, up 11008x4096; down 4096x11008} = 224 linear layers): the grouped
optimizer step of every layer (INT4 projection dequant, R = P~^T G on bf16 MFMA, Adam with
INT8 moments, U = alpha P~ N~ with the fused stochastic rounding into INT8 weights) plus the
layer-adaptive refresh test of the layers whose refresh falls due at that step (CosSim of the
stored projection with a new one, and the interval bookkeeping). Refreshes are staggered over
the initial interval of 25 steps, so about 224/25 layers are tested per step.

All inputs are synthetic and resident in HBM before timing starts (gradients ~N(0, 1e-4^2) in
bf16, INT8 weights with group scales 1e-3, projections from seeded QR quantized to INT4).
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA
# Vector ALU issue rate of MI355X: 256 CUs x 4 SIMDs x 16 lanes per cycle (a 64-lane
# instruction takes 4 cycles) x 2.4 GHz, in lane operations per second. The published fp32
# vector peak, 157.3 TFLOP/s, is this rate x 2 (an FMA) x 2 (packed fp32).
ALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
# Operations the method's arithmetic needs per element, counted one per fp32/int32 operation
# of the contract (a division, square root or 32 x 32 -> 64-bit multiply counts one):
#   rounding of one weight: U = alpha*S, a = U*inv, w to fp32, t = w + a, the 16 random bits
#   to fp32, d = t + u, floor, clamp (8), plus Philox4x32-10 for 8 weights: 10 rounds of two
#   multiplies and two three-way XORs, 40 per 8 weights (5);
SR_OPS_PER_WEIGHT = 8 + 5
#   Adam on one element of R: two moment dequantizations (4), m1 (3), v1 (4), the two bias
#   corrections (2), sqrt, + eps, lr * m^, the division (4), the two absmax steps (2), the
#   two requantizations (6), N~ to bf16 (1);
ADAM_OPS_PER_ELEM = 26
#   INT4 dequantization of one P element: code to fp32, one fma (2).
DEQUANT_OPS_PER_ELEM = 2
DELTA0 = 25                    # initial refresh interval (200 steps / 8)
GAMMA = 0.4


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


_HOST_QR = {}


def projection(cfg, L, r, tag, torch, WL, dev, fast):
    """An orthonormal m x r projection for layer L: the Q of a seeded Gaussian, by QR on the
    device, or with `fast` (profiling runs) by numpy QR on the host, computed once per shape and
    tag and shared by the layers of that shape, so that no device QR (rocsolver) runs inside a
    profiled process."""
    if not fast:
        return WL.orthonormal_device(cfg, L, r, tag=tag, device=dev)
    key = (L.m, r, tag)
    if key not in _HOST_QR:
        _HOST_QR[key] = torch.from_numpy(WL.orthonormal_f32(cfg, L, r, tag=tag))
    return _HOST_QR[key].to(dev)


def build_layer_set(cfg, r, G_list, W_list, Ws_list, torch, B, WL, fast=False, fmt="int4"):
    """Per-layer optimizer state for rank r (projections stored in format fmt, moments)
    sharing G and W."""
    layers, pnew = [], []
    dev = torch.device("cuda:0")
    shape_new = {}
    for k, L in enumerate(cfg.layers):
        P = projection(cfg, L, r, WL.TAG_P, torch, WL, dev, fast)
        Pq, Ps = B.quantize_proj(P, fmt=fmt)
        del P
        ng = B.n_groups(r * L.n)
        layers.append(B.LayerTensors(
            layer_id=L.layer_id, G=G_list[k], Wq=W_list[k], Ws=Ws_list[k], Pq=Pq, Ps=Ps,
            Mq=torch.zeros((r, L.n), dtype=torch.int8, device=dev),
            Ms=torch.zeros(ng, dtype=torch.float32, device=dev),
            Vq=torch.zeros((r, L.n), dtype=torch.int8, device=dev),
            Vs=torch.zeros(ng, dtype=torch.float32, device=dev), r=r, p_format=fmt))
        # one candidate "new" projection per distinct shape stands in for the SVD result
        if (L.m, L.n) not in shape_new:
            Pn = projection(cfg, L, r, WL.TAG_PNEW, torch, WL, dev, fast)
            shape_new[(L.m, L.n)] = B.quantize_proj(Pn, fmt=fmt)
            del Pn
        pnew.append(shape_new[(L.m, L.n)])
    torch.cuda.synchronize()
    return layers, pnew


class Variant:
    """One rank variant of the layer set: plans, refresh schedules and scratch.

    G_sets holds one or more gradient sets (each a list with one bf16 G per layer, all
    resident in HBM); step t uses set t mod len(G_sets), through a plan of its own (plans
    differ only in their G pointers and share the workspace), so that the moments see a fresh
    gradient each step instead of settling on a repeated one."""

    def __init__(self, cfg, r, G_sets, W_list, Ws_list, torch, B, WL, fast=False, fmt="int4",
                 dequant="auto", keep_proj=False, window=0):
        """window > 0: the step runs as consecutive plans of `window` layers each, sharing one
        workspace sized for the largest (the step-transient N~ and bf16 P~ of only `window`
        layers exist at a time)."""
        self.cfg, self.r, self.fmt = cfg, r, fmt
        self.torch, self.B = torch, B
        t0 = time.time()
        self.layers, self.pnew = build_layer_set(cfg, r, G_sets[0], W_list, Ws_list, torch, B,
                                                 WL, fast, fmt)
        hp = dict(lr=cfg.lr, beta1=cfg.beta1, beta2=cfg.beta2, eps=cfg.eps, alpha=cfg.alpha)
        nl = len(self.layers)
        w = window if 0 < window < nl else nl
        self.window = w if w < nl else None
        self.chunks = [(a, min(nl, a + w)) for a in range(0, nl, w)]
        self.plans = []     # per gradient set: one plan per chunk of layers
        for Gs in G_sets:
            lt = [dataclasses.replace(L, G=G) for L, G in zip(self.layers, Gs)]
            self.plans.append([B.Plan(lt[a:b], hp=hp, dequant=dequant) for a, b in self.chunks])
        self.all_plans = [p for ps in self.plans for p in ps]
        self.plan = self.plans[0][0]
        self.workspace_bytes = max(p.workspace_bytes for p in self.all_plans)
        # keep_proj (comparison runs only): with the separate dequant pass, keep the bf16
        # projections between steps and re-dequantize only the layers a refresh test replaced.
        # The step proper dequantizes every projection every step.
        self.keep_proj = keep_proj and len(self.all_plans) == 1
        if self.keep_proj:
            self.plan.cache_proj(True)
        self.ws = B.alloc_workspace(self.workspace_bytes)
        self.cws = B.alloc_workspace(B.cossim_batch_workspace_bytes(r, 32))
        self.cs_out = torch.zeros(len(self.layers), dtype=torch.float32, device="cuda")
        # staggered schedules: layer l had its first refresh at (l mod 25) - 25
        self.sched = []
        for k in range(len(self.layers)):
            s = B.Schedule(DELTA0, GAMMA)
            s.refresh(k % DELTA0 - DELTA0, None)
            self.sched.append(s)
        self.t = 0
        self.tests = 0
        log(f"rank {r}: {len(self.layers)} layers ready in {time.time() - t0:.1f}s, "
            f"workspace {self.plan.workspace_bytes / 2**30:.2f} GiB")

    def step(self):
        """One full step: grouped optimizer step, then the due refresh tests. A layer due
        for a refresh gets a new projection, which the next step dequantizes again."""
        self.t += 1
        t = self.t
        for p in self.plans[t % len(self.plans)]:
            p.step(t, 1234, self.ws)
        due = [k for k, s in enumerate(self.sched) if s.due(t)]
        if due:
            pairs = [(*self.pnew[k], self.layers[k].Pq, self.layers[k].Ps, self.layers[k].m,
                      self.fmt) for k in due]
            self.B.cossim_batch(pairs, self.r, self.cs_out, workspace=self.cws)
        vals = self.cs_out[: len(due)].cpu().tolist() if due else []
        for k, v in zip(due, vals):
            self.sched[k].refresh(t, v)
            if self.keep_proj:
                self.plan.proj_changed(k)
        self.tests += len(due)

    def time_steps(self, steps, warmup):
        torch = self.torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        for p in self.all_plans:
            p.enable_timing(steps)
        self.tests = 0
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize()
        evs[0].record()
        for i in range(steps):
            self.step()
            evs[i + 1].record()
        torch.cuda.synchronize()
        total_ms = evs[0].elapsed_time(evs[-1])
        per = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(steps))
        self.step_pct = {q: round(per[min(steps - 1, int(round(f * (steps - 1))))], 4)
                         for q, f in (("p10", 0.1), ("median", 0.5), ("p90", 0.9))}
        acc = [0.0] * 4     # summed over the chunks of a step, averaged over the steps
        for p in self.all_plans:
            kms_p, n_p = p.kernel_times()
            acc = [a + k * n_p for a, k in zip(acc, kms_p)]
            p.enable_timing(0)
        kms = [a / steps for a in acc]
        return total_ms / steps, kms, self.tests / steps

    def close(self):
        for p in self.all_plans:
            p.close()

    def time_cossim(self, reps=5):
        """Latency (ms) of the batched refresh test for one layer of each shape and for a
        batch of nine layers (the per-step load of the staggered schedule)."""
        torch = self.torch
        out = {}
        for label, ks in (("1 layer", [0]), ("9 layers", list(range(9)))):
            if ks[-1] >= len(self.layers):   # a set of fewer layers has no nine-layer batch
                continue
            pairs = [(*self.pnew[k], self.layers[k].Pq, self.layers[k].Ps, self.layers[k].m,
                      self.fmt) for k in ks]
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            self.B.cossim_batch(pairs, self.r, self.cs_out, workspace=self.cws)
            e0.record()
            for _ in range(reps):
                self.B.cossim_batch(pairs, self.r, self.cs_out, workspace=self.cws)
            e1.record()
            torch.cuda.synchronize()
            out[label] = round(e0.elapsed_time(e1) / reps, 4)
        return out


KERNELS = ("qg_dequant", "qg_project", "qg_adam", "qg_backproject")


def describe_layers(cfg) -> str:
    """The layer set in words: LLaMA-shaped sets by their per-block shapes (q, k, v, o d x d;
    gate, up f x d; down d x f), anything else by its shape counts."""
    shapes = [(L.m, L.n) for L in cfg.layers]
    if len(shapes) == 1:
        return f"one {shapes[0][0]}x{shapes[0][1]} layer"
    if len(shapes) % 7 == 0:
        d, f = shapes[0][0], shapes[4][0]
        block = [(d, d)] * 4 + [(f, d)] * 2 + [(d, f)]
        if shapes == block * (len(shapes) // 7):
            name = {4096: "LLaMA-7B", 2048: "LLaMA-1B", 512: "LLaMA-60M"}.get(d, "LLaMA")
            return (f"{name}-shaped layer set, {len(shapes)} layers ({len(shapes) // 7} x "
                    f"q,k,v,o {d}x{d}; gate,up {f}x{d}; down {d}x{f})")
    counts = {}
    for sh in shapes:
        counts[sh] = counts.get(sh, 0) + 1
    return f"{len(shapes)} layers (" + "; ".join(f"{c} x {m}x{n}" for (m, n), c in counts.items()) + ")"


def fused_adam(cfg):
    """The grouped step runs Adam inside the projection kernel when every layer's rows are
    whole 256-element groups (the 7B sets: n in {4096, 11008}) and the layer set fills the chip
    with one K split per layer."""
    return all(L.n % 256 == 0 for L in cfg.layers)


def inline_dequant(fmt, r, mode):
    """Whether the library dequantizes the INT4 projections of rank r inside its MFMA kernels
    (the rule of qg_dequant_mode: INLINE asked for, INT4, r % 32 == 0 and r % 128 == 0 or
    256 % r == 0; AUTO is the separate pass)."""
    return fmt == "int4" and mode == "inline" and r % 32 == 0 and (r % 128 == 0 or 256 % r == 0)


def algorithmic(cfg, r, fmt="int4", inline=False):
    """FLOPs and bytes the method must do per step, split by the kernel that does them (in
    launch order: INT4 dequant of P, projection, Adam, back-projection + rounding). Bytes
    count each algorithmic input once and each output once: P (INT4 + fp32 scale per 256)
    once, G once, M and V (INT8 + scales) read and written, W (INT8) read and written with
    its scales read. Workspace round trips (R partials, N~, the bf16 copy of P~) are not
    algorithmic and are not counted. When Adam runs inside the projection kernel, its bytes
    are that kernel's."""
    mn = sum(L.m * L.n for L in cfg.layers)
    mr = sum(L.m * r for L in cfg.layers)
    rn = sum(r * L.n for L in cfg.layers)
    adam = 4.0 * rn + 4.0 * 4.0 * rn / 256.0          # M, V in and out + their scales
    fused = fused_adam(cfg)
    flops = (0.0, 2.0 * r * mn, 0.0, 2.0 * r * mn)
    p_bytes = {"int4": 0.5 * mr + mr / 64.0, "int8": mr + mr / 64.0, "bf16": 0.0}[fmt]
    # P codes + scales: the dequant pass's input, or read by the projection kernel when the
    # MFMA kernels dequantize it themselves (bf16: read directly, not counted)
    nbytes = (0.0 if inline else p_bytes,
              2.0 * mn + (adam if fused else 0.0) + (p_bytes if inline else 0.0),
              0.0 if fused else adam,
              2.0 * mn + mn / 64.0)                   # W in and out + W scales
    deq = 0.0 if fmt == "bf16" else DEQUANT_OPS_PER_ELEM * mr
    ops = (0.0 if inline else deq,
           (ADAM_OPS_PER_ELEM * rn if fused else 0.0) + (deq if inline else 0.0),
           0.0 if fused else ADAM_OPS_PER_ELEM * rn,
           SR_OPS_PER_WEIGHT * mn)
    return dict(mn=mn, flops=flops, bytes=nbytes, ops=ops, fused_adam=fused)


def roofline(cfg, r, kms, fmt="int4", inline=False, launches=1):
    """kms: each kernel's time per step; launches: the launches of each kernel per step (the
    plans of a windowed step), each doing an equal share of the set's work."""
    a = algorithmic(cfg, r, fmt, inline)
    names = KERNELS
    k = max(range(4), key=lambda i: kms[i])            # dominant kernel
    sec = kms[k] / 1e3
    # the counter summaries hold one launch over the whole set
    traffic = measured_traffic(cfg.key, names[k]) if fmt == "int4" and launches == 1 else None
    if k == 1 and a["fused_adam"]:
        names = list(names)
        names[1] = "qg_project (+ Adam)"
    # the binding unit: the largest of the kernel's lower-bound times on HBM, the bf16 matrix
    # cores and the vector ALUs
    t_hbm = a["bytes"][k] / (HBM_PEAK_GBS * 1e9)
    t_mfma = a["flops"][k] / (BF16_MFMA_PEAK_TFLOPS * 1e12)
    t_alu = a["ops"][k] / (ALU_PEAK_TOPS * 1e12)
    common = dict(kernel=names[k], traffic=traffic, ms_per_launch=round(kms[k] / launches, 4),
                  **({"launches_per_step": launches} if launches > 1 else {}),
                  lower_bound_ms={"hbm": round(t_hbm * 1e3, 4), "mfma": round(t_mfma * 1e3, 4),
                                  "alu": round(t_alu * 1e3, 4)})
    if t_mfma >= max(t_hbm, t_alu):
        ach = a["flops"][k] / sec / 1e12
        return dict(bound="mfma", achieved=round(ach, 2), peak=BF16_MFMA_PEAK_TFLOPS,
                    unit="TFLOP/s", frac=round(ach / BF16_MFMA_PEAK_TFLOPS, 4), **common)
    if t_alu >= t_hbm:
        ach = a["ops"][k] / sec / 1e12
        return dict(bound="alu", achieved=round(ach, 2), peak=round(ALU_PEAK_TOPS, 2),
                    unit="TOP/s", frac=round(ach / ALU_PEAK_TOPS, 4), **common)
    ach = a["bytes"][k] / sec / 1e9
    return dict(bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(ach / HBM_PEAK_GBS, 4), **common)


KERNEL_SOURCES = ("qg_kernels.hip", "qg_gemm.hpp", "qg_device.hpp", "qg_kernels.hpp")


def kernel_source_hash():
    """sha256 over the code of the step kernels' sources (comments and blank lines
    dropped): HBM traffic figures taken by a counter run apply only while this hash is
    unchanged."""
    import hashlib
    import re
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "quantized_rank_gradient_amd", "csrc", name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        lines = [ln.split("//")[0].rstrip() for ln in text.splitlines()]
        h.update("\n".join(ln for ln in lines if ln.strip()).encode())
    return h.hexdigest()[:16]


def measured_traffic(config_key, kernel):
    """HBM bytes per launch of `kernel` on `config_key` from the counter summary in
    profiles/traffic.json (FETCH_SIZE + WRITE_SIZE, each scaled by what the same counter
    reads for a copy of known size), or None when absent or taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            doc = json.load(f)
    except (OSError, ValueError):
        return None
    if doc.get("kernel_source_hash") != kernel_source_hash():
        return None
    ent = doc.get("configs", {}).get(config_key, {}).get(kernel)
    return None if ent is None else float(ent["hbm_bytes"])


def refresh_ms(torch, B, WL, cfg, reps=10):
    """Time of one projection refresh per distinct 7B shape at rank cfg.r: the library's
    (qgalore_refresh_proj, INT4 output included) against the same randomized range finder
    in torch (plus the library's INT4 quantization), on a drifting-workload gradient whose
    leading subspace has the refresh's rank."""
    out = {}
    dev = torch.device("cuda:0")
    seen = set()
    for L in cfg.layers:
        if (L.m, L.n) in seen:
            continue
        seen.add((L.m, L.n))
        G = WL.drift_gradient_device(cfg, L, WL.drift_basis_device(cfg, L, device=dev), 0.01, 3)
        k = cfg.r + 8
        Om = WL.sketch_device(cfg, L, k, 3, device=dev)
        ws = B.alloc_workspace(B.refresh_workspace_bytes(L.m, L.n, cfg.r, 8))
        for _ in range(2):
            B.refresh_proj(G, cfg.r, Om, workspace=ws)
            B.quantize_proj(WL.top_subspace_device(cfg, L, G, cfg.r, 3))
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            B.refresh_proj(G, cfg.r, Om, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        lib = e0.elapsed_time(e1) / reps
        t0 = time.time()
        for _ in range(reps):
            B.quantize_proj(WL.top_subspace_device(cfg, L, G, cfg.r, 3))
        torch.cuda.synchronize()
        ref = (time.time() - t0) / reps * 1e3
        out[f"{L.m}x{L.n}"] = {"library": round(lib, 3), "torch": round(ref, 3)}
        del G, Om, ws
    return out


def linear_bench(torch, B, WL, T, reps):
    """The three products of an INT8-weight linear layer for each distinct 7B shape at T
    tokens: per-call time and TFLOP/s of the library kernels (dequantization fused), against
    torch doing the same with an explicit dequantization to bf16 and hipBLASLt products."""
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(17)
    shapes = sorted({(L.m, L.n) for L in WL.CONFIGS["llama7b_r1024"].layers})
    rows = {}
    tot_flop = tot_lib = tot_ref = 0.0
    count = {}
    for L in WL.CONFIGS["llama7b_r1024"].layers:
        count[(L.m, L.n)] = count.get((L.m, L.n), 0) + 1

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    for (m, n) in shapes:
        Wq = torch.randint(-127, 128, (m, n), generator=gen, device=dev, dtype=torch.int8)
        Ws = torch.rand(B.n_groups(m * n), generator=gen, device=dev) * 1e-3 + 5e-4
        X = torch.randn((T, n), generator=gen, device=dev).to(torch.bfloat16)
        dY = torch.randn((T, m), generator=gen, device=dev).to(torch.bfloat16)
        Y = torch.empty((T, m), dtype=torch.bfloat16, device=dev)
        dX = torch.empty((T, n), dtype=torch.bfloat16, device=dev)
        G = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        flop = 2.0 * T * m * n

        def deq():
            return (Wq.float().reshape(-1)[: m * n].reshape(-1, 256) *
                    Ws[:, None]).reshape(m, n).to(torch.bfloat16) if (m * n) % 256 == 0 else None
        lib = [timed(lambda: B.int8_linear_fwd(X, Wq, Ws, out=Y)),
               timed(lambda: B.int8_linear_bwd_data(dY, Wq, Ws, out=dX)),
               timed(lambda: B.linear_bwd_weight(dY, X, out=G))]
        ref = [timed(lambda: torch.matmul(X, deq().t())),
               timed(lambda: torch.matmul(dY, deq())),
               timed(lambda: torch.matmul(dY.t(), X))]
        key = f"{m}x{n}"
        rows[key] = {"library_ms": [round(x, 4) for x in lib],
                     "torch_dequant_matmul_ms": [round(x, 4) for x in ref],
                     "library_tflops": [round(flop / (x * 1e-3) / 1e12, 1) for x in lib]}
        c = count[(m, n)]
        tot_flop += 3 * flop * c
        tot_lib += sum(lib) * c
        tot_ref += sum(ref) * c
        del Wq, Ws, X, dY, Y, dX, G
        torch.cuda.empty_cache()
    return {"metric": "INT8-weight linear layer products (forward, data and weight gradients), "
                      "LLaMA-7B layer set", "tokens": T,
            "value": round(tot_flop / (tot_lib * 1e-3) / 1e12, 1), "unit": "TFLOP/s",
            "frac_of_bf16_peak": round(tot_flop / (tot_lib * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
            "layer_set_ms": round(tot_lib, 2), "torch_layer_set_ms": round(tot_ref, 2),
            "shapes": rows}


def copy_bandwidth(torch, gib=2.0, reps=5):
    """Read+write GB/s of a device-to-device copy of `gib` GiB (torch's copy kernel): the
    achievable HBM rate beside the 8 TB/s peak, and the copy of known size against which the
    memory counters are calibrated."""
    n = int(gib * 2**30)
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    # a read-only pass (a sum over the source) and a write-only one (a fill of the
    # destination) of the same size: the second and third kernels of known traffic that the
    # counters' calibration is checked on (not timed: torch's sum makes more than one pass)
    src32 = src.view(torch.int32)
    for _ in range(reps):
        src32.sum()
        dst.fill_(2)
    torch.cuda.synchronize()
    del src, dst, src32
    torch.cuda.empty_cache()
    return dict(bytes_per_copy=2 * n, ms=round(ms, 4), gbs=round(2 * n / (ms / 1e3) / 1e9, 1))


def mfma_sustained(torch, B, seconds=1.5):
    """TFLOP/s of the library's MFMA calibration kernel (bf16 32x32x16 products from register
    operands, no memory traffic) held for about `seconds` each on random operands like the
    step's (bf16 ~N(0, 0.05^2)) and on constant ones: the rate the matrix cores sustain
    under the clock the load allows, beside the published dense peak that the roofline
    fraction is taken against."""
    out = {"random_operands": mfma_hold(torch, B, seconds)["tflops"],
           "constant_operands": mfma_hold(torch, B, seconds, constant=True)["tflops"],
           "seconds_each": seconds, "unit": "TFLOP/s"}
    return out


def mfma_hold(torch, B, seconds, grid=1024, iters=2000, constant=False):
    """Runs the MFMA calibration kernel on random (or constant) bf16 operands for about
    `seconds` and returns the rate it sustained; with board power and clock readings taken
    beside it, the power-limited rate of bare matrix work."""
    buf = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
    if constant:
        ops = torch.full((1 << 23,), 0.01, device="cuda", dtype=torch.bfloat16)
    else:
        gen = torch.Generator(device="cuda")
        gen.manual_seed(20240711)
        ops = (torch.randn(1 << 23, generator=gen, device="cuda") * 0.05).to(torch.bfloat16)
    flops = B.mfma_probe(ops, buf, grid, iters)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    B.mfma_probe(ops, buf, grid, iters)
    e1.record()
    torch.cuda.synchronize()
    launches = max(1, int(seconds * 1e3 / e0.elapsed_time(e1)))
    e0.record()
    for _ in range(launches):
        B.mfma_probe(ops, buf, grid, iters)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    return {"mfma_probe": "constant bf16 operands" if constant else "random bf16 operands",
            "launches": launches, "seconds": round(ms / 1e3, 2),
            "tflops": round(flops * launches / (ms / 1e3) / 1e12, 1)}


def library_gemm_ms(torch, cfg, r, reps=20):
    """torch (hipBLASLt) bf16 matmuls with the shapes of the two contractions, summed over
    the layer set: R = P^T G with P^T stored contiguous, and P N (no fused epilogues). A
    point of comparison for the MFMA kernels, not part of a step."""
    by_shape = {}
    for L in cfg.layers:
        by_shape[(L.m, L.n)] = by_shape.get((L.m, L.n), 0) + 1
    total = [0.0, 0.0]
    for (m, n), count in by_shape.items():
        P = torch.randn(m, r, device="cuda", dtype=torch.bfloat16)
        PT = P.t().contiguous()
        G = torch.randn(m, n, device="cuda", dtype=torch.bfloat16)
        N = torch.randn(r, n, device="cuda", dtype=torch.bfloat16)
        for k, fn in enumerate((lambda: torch.matmul(PT, G), lambda: torch.matmul(P, N))):
            for _ in range(3):
                fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            total[k] += e0.elapsed_time(e1) / reps * count
        del P, PT, G, N
    torch.cuda.empty_cache()
    return dict(projection_ms=round(total[0], 3), backprojection_ms=round(total[1], 3))


def _oracle_worker(layer_ids, barrier, out):
    """One process of the CPU baseline: builds the inputs of its layers (not timed), waits for
    every worker, then runs one oracle step per layer with one BLAS thread."""
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass
    from oracle import qgalore_oracle as O
    from quantized_rank_gradient_amd import workloads as WL
    cfg = WL.CONFIGS["llama7b_r1024"]
    h = O.Hyper(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.alpha)
    jobs = []
    for k in layer_ids:
        L = cfg.layers[k]
        P = WL.orthonormal_f32(cfg, L, cfg.r)
        Pq, Ps = O.quantize_proj(P)
        Mq, Ms, Vq, Vs = WL.zero_moments(cfg.r, L.n)
        st = O.LayerState(L.m, L.n, cfg.r, L.layer_id, WL.weights_int8(cfg, L),
                          WL.weight_scales(cfg, L), Pq, Ps, Mq, Ms, Vq, Vs)
        jobs.append((st, WL.gradient_bf16(cfg, L, 1), L.m * L.n))
    barrier.wait()
    t0 = time.time()
    for st, G, _ in jobs:
        O.qgalore_step(st, G, 1, 1234, h)
    t1 = time.time()
    out.put((sum(e for _, _, e in jobs), t0, t1))


def cpu_baseline(max_layers=8):
    """The oracle, as it stands, on a bounded sample of the 7B set at rank 1024: one full oracle
    step on each of the first attention layers (4096 x 4096: q, k, v, o of blocks 0, 1, ...),
    one layer per worker process, as many workers as host cores this process may run on (at
    most max_layers), each with one BLAS thread. Every worker builds its inputs first; the timed
    span runs from the common start to the last worker's end. Call it before the process touches
    the GPU: the workers are forked."""
    import multiprocessing as mp
    from quantized_rank_gradient_amd import workloads as WL
    host = len(os.sched_getaffinity(0))
    workers = max(1, min(host, max_layers))
    cfg = WL.CONFIGS["llama7b_r1024"]
    sample = [k for k, L in enumerate(cfg.layers) if L.m == L.n][:workers]
    nlayers = len(sample)
    ctx = mp.get_context("fork")
    barrier = ctx.Barrier(workers)
    out = ctx.Queue()
    parts = [[k] for k in sample]
    procs = [ctx.Process(target=_oracle_worker, args=(parts[w], barrier, out))
             for w in range(workers)]
    for pr in procs:
        pr.start()
    res = [out.get() for _ in procs]
    for pr in procs:
        pr.join()
    elems = sum(e for e, _, _ in res)
    span = max(t1 for _, _, t1 in res) - min(t0 for _, t0, _ in res)
    busy = sum(t1 - t0 for _, t0, t1 in res)
    return dict(value=round(elems / span, 1), unit="weight elems/s", cores=workers,
                kind="oracle", host_cores=host, blas_threads_per_worker=1,
                seconds=round(span, 2), cpu_seconds=round(busy, 2),
                sample=f"one full oracle step of each of {nlayers} rank-1024 4096x4096 layers "
                       f"(q, k, v, o of the first blocks) of the 7B set ({elems} weight "
                       f"elements), one per worker process; input generation not timed")


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="llama7b_r1024")
    ap.add_argument("--secondary", default="llama7b_r128",
                    help="a second rank variant reported alongside ('none' to skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-gib", type=float, default=2.0,
                    help="size of the device copy timed for the achievable HBM rate (0: skip)")
    ap.add_argument("--schedule", action="store_true",
                    help="instead: run the adaptive refresh schedule (7B shapes, rank 128, 200 "
                         "steps of drifting gradients) and report the SVDs it saves")
    ap.add_argument("--linear", action="store_true",
                    help="instead: time the INT8-weight linear products (forward, data and "
                         "weight gradients) on the 7B layer shapes")
    ap.add_argument("--mfma-seconds", type=float, default=0.0,
                    help="instead: run the MFMA calibration kernel on random operands for this "
                         "many seconds (board power and clock readings beside it)")
    ap.add_argument("--refresh-only", action="store_true",
                    help="instead: time one projection refresh per 7B shape (library vs torch)")
    ap.add_argument("--refresh-ranks", default="128",
                    help="with --refresh-only: the ranks timed (comma-separated; 8 extra "
                         "sketch columns each)")
    ap.add_argument("--tokens", type=int, default=8192,
                    help="with --linear: tokens per batch (batch x sequence length)")
    ap.add_argument("--refresh", default="library", choices=("library", "torch"),
                    help="with --schedule: who computes the new projections (torch: the same "
                         "randomized range finder in torch, for comparison)")
    ap.add_argument("--p-format", default="int4", choices=("int4", "int8", "bf16"),
                    help="storage format of the projections (int8, bf16: comparison runs)")
    ap.add_argument("--library-gemm", action="store_true",
                    help="also time torch bf16 matmuls of the same shapes (comparison only)")
    ap.add_argument("--fast-setup", action="store_true",
                    help="profiling runs: projections from numpy QR on the host, one per shape "
                         "(no device QR in the profiled process)")
    ap.add_argument("--dequant", default="auto", choices=("auto", "inline", "pass"),
                    help="where INT4 projections are dequantized: in the MFMA kernels' stagers "
                         "(inline), by a separate pass into the workspace (pass), or the "
                         "library's choice (auto)")
    ap.add_argument("--window", type=int, default=0,
                    help="run the step as consecutive plans of this many layers sharing one "
                         "workspace (0: one plan over the whole set)")
    ap.add_argument("--keep-proj", action="store_true",
                    help="comparison: with the separate pass, keep dequantized projections "
                         "between steps (only refreshed layers are dequantized again)")
    ap.add_argument("--g-sets", type=int, default=4,
                    help="gradient sets resident in HBM, used in turn by the timed steps")
    ap.add_argument("--configs", default="single256,llama60m,llama1b,llama7b_r1024_window56",
                    help="the other layer sets timed and reported under 'configs' "
                         "(comma-separated; 'none' to skip; <set>_window<N>: that set's step "
                         "in plans of N layers sharing one workspace)")
    ap.add_argument("--config-steps", type=int, default=20,
                    help="timed steps of each of the other layer sets")
    ap.add_argument("--no-schedule", action="store_true",
                    help="skip the adaptive-schedule run (200 steps) reported under 'configs'")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the Q-GaLore step runs on a single MI355X here; "
              "multi-GPU runs are not part of this benchmark", file=sys.stderr)
        sys.exit(2)

    # the oracle's baseline runs first, in forked worker processes, before the GPU is touched
    cpu = None
    if not (args.no_cpu_baseline or args.schedule or args.linear or args.refresh_only
            or args.mfma_seconds > 0):
        log("timing the CPU oracle ...")
        cpu = cpu_baseline()
        log(f"cpu baseline: {json.dumps(cpu)}")

    import torch
    from quantized_rank_gradient_amd import binding as B
    from quantized_rank_gradient_amd import workloads as WL
    B.lib()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)

    if args.schedule:
        from quantized_rank_gradient_amd.schedule_run import ScheduleRun
        scfg = WL.CONFIGS["schedule7b"]
        rf = refresh_ms(torch, B, WL, scfg)
        log(f"one refresh (rank {scfg.r}): {json.dumps(rf)}")
        t0 = time.time()
        run = ScheduleRun(scfg, refresh=args.refresh)
        log(f"schedule workload ready in {time.time() - t0:.1f}s")
        t0 = time.time()
        summ = run.run()
        run.close()
        counts = summ.pop("per_layer_counts")
        hist = {str(c): counts.count(c) for c in sorted(set(counts))}
        print(json.dumps({
            "metric": "adaptive refresh schedule: SVDs saved against a fixed interval",
            "value": summ["svds_saved"], "unit": "fraction", "higher_is_better": True,
            "data": "synthetic",
            "config": {"workload": "schedule7b: LLaMA-7B-shaped layer set, 224 layers, rank 128, "
                                   "200 steps, drifting low-rank gradients (0 .. 0.05 rad/step), "
                                   "interval 25 doubling when CosSim > 0.4"},
            **summ, "layers_by_refresh_count": hist, "refresh_ms": rf,
            "wall_s": round(time.time() - t0, 1)}), flush=True)
        return

    if args.linear:
        print(json.dumps(linear_bench(torch, B, WL, args.tokens, args.steps)), flush=True)
        return
    if args.mfma_seconds > 0:
        print(json.dumps(mfma_hold(torch, B, args.mfma_seconds)), flush=True)
        return
    if args.refresh_only:
        scfg = WL.CONFIGS["schedule7b"]
        ranks = [int(x) for x in args.refresh_ranks.split(",")]
        print(json.dumps({"metric": "projection refresh time (8 extra columns, 2 power "
                                    "iterations): library vs torch range finder",
                          "unit": "ms",
                          "ranks": {str(r): refresh_ms(torch, B, WL,
                                                       dataclasses.replace(scfg, r=r))
                                    for r in ranks}}), flush=True)
        return

    cfg = WL.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    copy = copy_bandwidth(torch, args.copy_gib) if args.copy_gib > 0 else None
    if copy:
        log(f"device copy: {json.dumps(copy)}")
    sustained = mfma_sustained(torch, B) if args.copy_gib > 0 else None
    if sustained:
        log(f"sustained MFMA rate: {json.dumps(sustained)}")

    results = run_layer_set(args, torch, B, WL, cfg,
                            None if args.secondary == "none" else WL.CONFIGS[args.secondary],
                            args.g_sets, args.steps, args.warmup)
    main_res = results[0]
    line = {
        "metric": "Q-GaLore step: weight elems updated/s + % bf16-MFMA/HBM roofline, 7B layer set",
        "value": round(main_res["value"], 1),
        "unit": "weight elems/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.key}: {describe_layers(cfg)}, rank {cfg.r}, "
                        f"one full optimizer step + due refresh tests",
            "layers": len(cfg.layers), "rank": cfg.r, "weight_elems": algorithmic(cfg, cfg.r)["mn"],
            "projection_format": args.p_format,
            "gradient_sets": main_res["gradient_sets"],
            "parallelism": "single GPU",
        },
        **{k: main_res[k] for k in ("step_ms_percentiles", "tflops", "dequant", "window",
                                    "workspace_gib", "projection_gib",
                                    "kernel_ms", "optimizer_ms", "refresh_tests_per_step",
                                    "cossim_ms", "roofline")},
        "copy_gbs": copy["gbs"] if copy else None,
        "mfma_sustained": sustained,
    }
    if "library_gemm" in main_res:
        line["library_gemm"] = main_res["library_gemm"]
    subs = {}
    for r in results[1:]:
        subs[r["config"]] = r
    torch.cuda.empty_cache()
    if args.configs != "none":
        for key in args.configs.split(","):
            # "<set>_window<N>": the set's step in plans of N layers sharing one workspace
            m = re.fullmatch(r"(.+)_window(\d+)", key)
            c = WL.CONFIGS[m.group(1) if m else key]
            steps = c.steps if c.steps > 1 else args.config_steps
            subs[key] = run_layer_set(args, torch, B, WL, c, None, args.g_sets if m else 2, steps,
                                      args.warmup, window=int(m.group(2)) if m else None)[0]
            torch.cuda.empty_cache()
    if not args.no_schedule:
        subs["schedule7b"] = schedule_summary(torch, B, WL)
        torch.cuda.empty_cache()
    line["configs"] = subs
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


def run_layer_set(args, torch, B, WL, cfg, secondary, g_sets, steps, warmup, window=None):
    """Times the step on cfg's layer set (and on `secondary`, a rank variant with the same
    shapes, sharing its gradients and weights). Returns one result per variant. window: layers
    per plan for this run (None: --window)."""
    dev = torch.device("cuda:0")
    t0 = time.time()
    G_sets = [[WL.gradient_bf16_device(cfg, L, 1 + g, device=dev) for L in cfg.layers]
              for g in range(g_sets)]
    W_list, Ws_list = [], []
    for L in cfg.layers:
        W_list.append(WL.weights_int8_device(cfg, L, device=dev))
        Ws_list.append(torch.full((B.n_groups(L.m * L.n),), cfg.w_scale, dtype=torch.float32,
                                  device=dev))
    torch.cuda.synchronize()
    log(f"{cfg.key}: {g_sets} x {len(cfg.layers)} gradients and INT8 weights resident in "
        f"{time.time() - t0:.1f}s")
    variants = [(cfg, cfg.r)]
    if secondary is not None:
        assert [(L.m, L.n) for L in secondary.layers] == [(L.m, L.n) for L in cfg.layers]
        variants.append((secondary, secondary.r))
    results = []
    for vcfg, r in variants:
        v = Variant(vcfg, r, G_sets, W_list, Ws_list, torch, B, WL, args.fast_setup,
                    args.p_format, args.dequant, args.keep_proj,
                    args.window if window is None else window)
        ms, kms, tests = v.time_steps(steps, warmup)
        cs_ms = v.time_cossim()
        a = algorithmic(vcfg, r, args.p_format)
        inl = inline_dequant(args.p_format, r, args.dequant)
        kernel_ms = {nm: round(t, 4) for nm, t in zip(KERNELS, kms)}
        if inl:
            kernel_ms["qg_dequant"] = "in qg_project and qg_backproject"   # no separate launch
        if a["fused_adam"]:
            kernel_ms["qg_adam"] = "in qg_project"   # no separate launch
        if args.p_format == "bf16":
            kernel_ms["qg_dequant"] = "none (bf16 projection)"
        p_bytes = sum(int(L.Pq.numel() * L.Pq.element_size()) +
                      (int(L.Ps.numel() * 4) if L.Ps is not None else 0) for L in v.layers)
        res = dict(config=vcfg.key if window is None else f"{vcfg.key}_window{window}",
                   workload=f"{vcfg.key}: {describe_layers(vcfg)}, rank {r}"
                            + (f", in plans of {v.window} layers sharing one workspace"
                               if v.window else ""),
                   rank=r, steps=steps, ms_per_step=round(ms, 4),
                   step_ms_percentiles=v.step_pct,
                   value=a["mn"] / (ms / 1e3),
                   tflops=round(4.0 * r * a["mn"] / (ms / 1e3) / 1e12, 2),
                   gradient_sets=g_sets,
                   dequant=args.dequant + ("+keep" if v.keep_proj else ""),
                   window=v.window,
                   workspace_gib=round(v.workspace_bytes / 2**30, 3),
                   projection_gib=round(p_bytes / 2**30, 3),
                   kernel_ms=kernel_ms,
                   optimizer_ms=round(sum(kms), 4),
                   refresh_tests_per_step=round(tests, 2),
                   cossim_ms=cs_ms,
                   roofline=roofline(vcfg, r, kms, args.p_format, inl, len(v.chunks)))
        if args.library_gemm:
            res["library_gemm"] = library_gemm_ms(torch, vcfg, r)
        log(json.dumps(res))
        results.append(res)
        v.close()
        del v
        torch.cuda.empty_cache()
    del G_sets, W_list, Ws_list
    return results


def schedule_summary(torch, B, WL):
    """The adaptive refresh schedule on the drifting 7B workload (224 layers, rank 128, 200
    steps): refreshes by the library, similarity tests, the grouped step every step."""
    from quantized_rank_gradient_amd.schedule_run import ScheduleRun
    scfg = WL.CONFIGS["schedule7b"]
    t0 = time.time()
    run = ScheduleRun(scfg)
    setup = time.time() - t0
    t0 = time.time()
    summ = run.run()
    run.close()
    counts = summ.pop("per_layer_counts")
    return dict(workload="schedule7b: LLaMA-7B-shaped layer set, 224 layers, rank 128, 200 steps, "
                         "drifting low-rank gradients (0 .. 0.05 rad/step), interval 25 doubling "
                         "when CosSim > 0.4",
                **summ, layers_by_refresh_count={str(c): counts.count(c) for c in sorted(set(counts))},
                setup_s=round(setup, 1), wall_s=round(time.time() - t0, 1))


if __name__ == "__main__":
    main()
