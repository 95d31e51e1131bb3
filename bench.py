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
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA
DELTA0 = 25                    # initial refresh interval (200 steps / 8)
GAMMA = 0.4


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def projection(cfg, L, r, tag, torch, WL, dev, fast):
    if not fast:
        return WL.orthonormal_device(cfg, L, r, tag=tag, device=dev)
    # profiling runs: Gaussian columns scaled to unit expected norm (no QR on the device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(WL.torch_seed(cfg, L.layer_id, 0, tag))
    return torch.randn((L.m, r), generator=gen, device=dev) / (L.m ** 0.5)


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
    """One rank variant of the layer set: a plan, refresh schedules and scratch."""

    def __init__(self, cfg, r, G_list, W_list, Ws_list, torch, B, WL, fast=False, fmt="int4"):
        self.cfg, self.r, self.fmt = cfg, r, fmt
        self.torch, self.B = torch, B
        t0 = time.time()
        self.layers, self.pnew = build_layer_set(cfg, r, G_list, W_list, Ws_list, torch, B, WL,
                                                 fast, fmt)
        self.plan = B.Plan(self.layers, hp=dict(lr=cfg.lr, beta1=cfg.beta1, beta2=cfg.beta2,
                                                 eps=cfg.eps, alpha=cfg.alpha))
        # dequantized projections are kept between steps; a refresh replaces a layer's P, so
        # every tested layer is marked changed and dequantized again at the next step
        self.plan.cache_proj(True)
        self.ws = B.alloc_workspace(self.plan.workspace_bytes)
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
        self.plan.step(t, 1234, self.ws)
        due = [k for k, s in enumerate(self.sched) if s.due(t)]
        if due:
            pairs = [(*self.pnew[k], self.layers[k].Pq, self.layers[k].Ps, self.layers[k].m,
                      self.fmt) for k in due]
            self.B.cossim_batch(pairs, self.r, self.cs_out, workspace=self.cws)
        vals = self.cs_out[: len(due)].cpu().tolist() if due else []
        for k, v in zip(due, vals):
            self.sched[k].refresh(t, v)
            self.plan.proj_changed(k)
        self.tests += len(due)

    def time_steps(self, steps, warmup):
        torch = self.torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        self.plan.enable_timing(steps)
        self.tests = 0
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for _ in range(steps):
            self.step()
        end.record()
        torch.cuda.synchronize()
        total_ms = start.elapsed_time(end)
        kms, nrec = self.plan.kernel_times()
        self.plan.enable_timing(0)
        return total_ms / steps, kms, self.tests / steps

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


def algorithmic(cfg, r, fmt="int4"):
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
    nbytes = (p_bytes,                                # P codes + scales (bf16: no pass)
              2.0 * mn + (adam if fused else 0.0),    # G (bf16) [+ Adam]
              0.0 if fused else adam,
              2.0 * mn + mn / 64.0)                   # W in and out + W scales
    return dict(mn=mn, flops=flops, bytes=nbytes, fused_adam=fused)


def roofline(cfg, r, kms, fmt="int4"):
    a = algorithmic(cfg, r, fmt)
    names = KERNELS
    k = max(range(4), key=lambda i: kms[i])            # dominant kernel
    sec = kms[k] / 1e3
    traffic = measured_traffic(cfg.key, names[k]) if fmt == "int4" else None
    if k == 1 and a["fused_adam"]:
        names = list(names)
        names[1] = "qg_project (+ Adam)"
    intensity = a["flops"][k] / a["bytes"][k] if a["bytes"][k] else 0.0
    mfma_bound = intensity > BF16_MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if mfma_bound:
        ach = a["flops"][k] / sec / 1e12
        return dict(kernel=names[k], bound="mfma", achieved=round(ach, 2),
                    peak=BF16_MFMA_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(ach / BF16_MFMA_PEAK_TFLOPS, 4), traffic=traffic,
                    ms_per_launch=round(kms[k], 4))
    ach = a["bytes"][k] / sec / 1e9
    return dict(kernel=names[k], bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS,
                unit="GB/s", frac=round(ach / HBM_PEAK_GBS, 4), traffic=traffic,
                ms_per_launch=round(kms[k], 4))


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
    in torch (plus the library's INT4 quantization), on a drifting-workload gradient."""
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
    del src, dst
    torch.cuda.empty_cache()
    return dict(bytes_per_copy=2 * n, ms=round(ms, 4), gbs=round(2 * n / (ms / 1e3) / 1e9, 1))


def mfma_sustained(torch, B, grid=1024, iters=2000, reps=3):
    """TFLOP/s of the library's MFMA calibration kernel (bf16 32x32x16 products from register
    operands, no memory traffic) on random operands like the step's (bf16 ~N(0, 0.05^2)) and
    on constant ones: the rate the matrix cores sustain under the clock the load allows,
    beside the published dense peak that the roofline fraction is taken against."""
    out = {}
    buf = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20240711)
    for label, ops in (("random_operands", (torch.randn(1 << 23, generator=gen, device="cuda")
                                             * 0.05).to(torch.bfloat16)),
                       ("constant_operands", torch.full((1 << 23,), 0.01, device="cuda",
                                                        dtype=torch.bfloat16))):
        flops = B.mfma_probe(ops, buf, grid, iters)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            B.mfma_probe(ops, buf, grid, iters)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[label] = round(flops / (ms / 1e3) / 1e12, 1)
        del ops
    out["unit"] = "TFLOP/s"
    return out


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


def cpu_baseline(nlayers=7):
    """The oracle, as it stands, on the layers of block 0 (q, k, v, o, gate, up, down) at
    rank 1024: one full oracle step per layer."""
    import numpy as np
    from oracle import qgalore_oracle as O
    from quantized_rank_gradient_amd import workloads as WL
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = 1
    cfg = WL.CONFIGS["llama7b_r1024"]
    h = O.Hyper(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.alpha)
    dt, elems = 0.0, 0
    for L in cfg.layers[:nlayers]:
        P = WL.orthonormal_f32(cfg, L, cfg.r)
        Pq, Ps = O.quantize_proj(P)
        Mq, Ms, Vq, Vs = WL.zero_moments(cfg.r, L.n)
        st = O.LayerState(L.m, L.n, cfg.r, L.layer_id, WL.weights_int8(cfg, L),
                          WL.weight_scales(cfg, L), Pq, Ps, Mq, Ms, Vq, Vs)
        G = WL.gradient_bf16(cfg, L, 1)
        t0 = time.time()
        O.qgalore_step(st, G, 1, 1234, h)
        dt += time.time() - t0
        elems += L.m * L.n
    return dict(value=round(elems / dt, 1), unit="weight elems/s", cores=int(threads),
                kind="oracle", seconds=round(dt, 2),
                sample=f"one full oracle step of each of the {nlayers} rank-1024 layers of "
                       f"block 0 ({elems} weight elements); input generation not timed")


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
    ap.add_argument("--refresh-only", action="store_true",
                    help="instead: time one projection refresh per 7B shape (library vs torch)")
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
                    help="Gaussian stand-in projections instead of QR (profiling runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the Q-GaLore step runs on a single MI355X here; "
              "multi-GPU runs are not part of this benchmark", file=sys.stderr)
        sys.exit(2)

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
    if args.refresh_only:
        scfg = WL.CONFIGS["schedule7b"]
        print(json.dumps({"metric": "projection refresh time (rank 128, 8 extra columns, 2 power "
                                    "iterations): library vs torch range finder",
                          "unit": "ms", "shapes": refresh_ms(torch, B, WL, scfg)}), flush=True)
        return

    cfg = WL.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    copy = copy_bandwidth(torch, args.copy_gib) if args.copy_gib > 0 else None
    if copy:
        log(f"device copy: {json.dumps(copy)}")
    sustained = mfma_sustained(torch, B) if args.copy_gib > 0 else None
    if sustained:
        log(f"sustained MFMA rate: {json.dumps(sustained)}")
    t0 = time.time()
    G_list, W_list, Ws_list = [], [], []
    for L in cfg.layers:
        G_list.append(WL.gradient_bf16_device(cfg, L, 1, device=dev))
        W_list.append(WL.weights_int8_device(cfg, L, device=dev))
        Ws_list.append(torch.full((B.n_groups(L.m * L.n),), cfg.w_scale, dtype=torch.float32,
                                  device=dev))
    torch.cuda.synchronize()
    log(f"{len(cfg.layers)} gradients and INT8 weights resident in {time.time() - t0:.1f}s")

    variants = [(cfg, cfg.r)]
    if args.secondary != "none":
        sec = WL.CONFIGS[args.secondary]
        assert [(L.m, L.n) for L in sec.layers] == [(L.m, L.n) for L in cfg.layers]
        variants.append((sec, sec.r))

    results = []
    for vcfg, r in variants:
        v = Variant(vcfg, r, G_list, W_list, Ws_list, torch, B, WL, args.fast_setup,
                    args.p_format)
        ms, kms, tests = v.time_steps(args.steps, args.warmup)
        cs_ms = v.time_cossim()
        a = algorithmic(vcfg, r, args.p_format)
        kernel_ms = {nm: round(t, 4) for nm, t in zip(KERNELS, kms)}
        if a["fused_adam"]:
            kernel_ms["qg_adam"] = "in qg_project"   # no separate launch
        if args.p_format == "bf16":
            kernel_ms["qg_dequant"] = "none (bf16 projection)"
        res = dict(config=vcfg.key, rank=r, ms_per_step=round(ms, 4),
                   value=a["mn"] / (ms / 1e3),
                   tflops=round(4.0 * r * a["mn"] / (ms / 1e3) / 1e12, 2),
                   kernel_ms=kernel_ms,
                   optimizer_ms=round(sum(kms), 4),
                   refresh_tests_per_step=round(tests, 2),
                   cossim_ms=cs_ms,
                   roofline=roofline(vcfg, r, kms, args.p_format))
        if args.library_gemm:
            res["library_gemm"] = library_gemm_ms(torch, vcfg, r)
        log(json.dumps(res))
        results.append(res)
        v.plan.close()
        del v
        torch.cuda.empty_cache()

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
            "parallelism": "single GPU",
        },
        "tflops": main_res["tflops"],
        "kernel_ms": main_res["kernel_ms"],
        "optimizer_ms": main_res["optimizer_ms"],
        "refresh_tests_per_step": main_res["refresh_tests_per_step"],
        "cossim_ms": main_res["cossim_ms"],
        "roofline": main_res["roofline"],
        "copy_gbs": copy["gbs"] if copy else None,
        "mfma_sustained": sustained,
        "variants": {r["config"]: {k: r[k] for k in ("rank", "value", "ms_per_step", "tflops",
                                                    "kernel_ms", "optimizer_ms",
                                                    "refresh_tests_per_step",
                                                    "cossim_ms", "roofline")}
                     for r in results[1:]},
    }
    line["variants"] = {
        r["config"]: {**line["variants"][r["config"]],
                      **({"library_gemm": r["library_gemm"]} if "library_gemm" in r else {})}
        for r in results[1:]
    }
    if "library_gemm" in main_res:
        line["library_gemm"] = main_res["library_gemm"]
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on one layer ...")
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
