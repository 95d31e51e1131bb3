"""Host-only tests of the C ABI: the library loads, exports every declared entry point, and
rejects bad arguments with the documented status before touching HIP. No kernel runs here."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import qgalore_oracle as O
from quantized_rank_gradient_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qgalore.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qgalore_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = B.lib()
    names = declared_functions()
    assert len(names) >= 15
    for name in names:
        assert hasattr(L, name), name
    assert set(names) == set(B.EXPORTS), "binding and header disagree"
    assert L.qgalore_version().startswith(b"qgalore")


def test_struct_layouts_match_header_sizes(tmp_path):
    """The ctypes structs have the size and field offsets the C compiler gives the header's."""
    import subprocess
    fields = {"qg_layer_desc": (B.LayerDesc, [f[0] for f in B.LayerDesc._fields_]),
              "qg_layer": (B.Layer, [f[0] for f in B.Layer._fields_]),
              "qg_proj": (B.Proj, [f[0] for f in B.Proj._fields_]),
              "qg_sched": (B.Sched, [f[0] for f in B.Sched._fields_])}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "qgalore.h"', "int main(void) {"]
    for cname, (_, names) in fields.items():
        lines.append(f'  printf("%zu\\n", sizeof({cname}));')
        for nm in names:
            lines.append(f'  printf("%zu\\n", offsetof({cname}, {nm}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "sizes.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "sizes"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o",
                    str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True,
                                          text=True).stdout.split()]
    want = []
    for cname, (cls, names) in fields.items():
        want.append(ctypes.sizeof(cls))
        want += [getattr(cls, nm).offset for nm in names]
    assert got == want


def _desc(m=256, n=256, r=32, **kw):
    d = B.LayerDesc()
    d.m, d.n, d.r, d.layer_id = m, n, r, 0
    d.lr, d.beta1, d.beta2, d.eps, d.alpha = 1e-3, 0.9, 0.999, 1e-8, 0.25
    fake = 0x10000
    d.M_scale = d.V_scale = fake
    d.workspace = fake
    d.workspace_bytes = 1 << 40
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def _call(d, G=0x10000, W=0x10000, Ws=0x10000, Pq=0x10000, Ps=0x10000, M=0x10000, V=0x10000,
          step=1):
    return B.lib().qgalore_step(ctypes.byref(d), G, W, Ws, Pq, Ps, M, V, step, 1234)


def test_step_validation_codes_without_touching_the_device():
    assert _call(_desc(), G=None) == 1
    assert _call(_desc(M_scale=None)) == 1
    assert _call(_desc(r=0)) == 2
    assert _call(_desc(r=300, m=256)) == 2          # r > m
    assert _call(_desc(r=12)) == 2                  # r % 8 != 0
    assert _call(_desc(n=0)) == 2
    assert _call(_desc(), G=0x10001) == 3            # misaligned
    assert _call(_desc(), Ws=0x10002) == 3
    assert _call(_desc(), step=0) == 5
    assert _call(_desc(), step=1 << 32) == 5
    assert _call(_desc(beta1=1.0)) == 5
    assert _call(_desc(eps=float("nan"))) == 5
    assert _call(_desc(workspace_bytes=16)) == 4
    assert _call(_desc(workspace=None)) == 1
    # m*r past 2^29 (r > n is allowed, so m*n and r*n alone do not bound the projection)
    assert _call(_desc(m=65536, n=8, r=32768)) == 2
    assert _call(_desc(m=65536, n=8, r=8192), G=None) == 1
    assert B.lib().qgalore_workspace_bytes(65536, 8, 32768) == 0
    assert B.lib().qgalore_quantize_proj(0x10000, 65536, 16384, 0x10000, 0x10000, None) == 2
    assert B.lib().qgalore_quantize_proj_int8(0x10000, 65536, 16384, 0x10000, 0x10000,
                                              None) == 2


def test_workspace_size_query():
    # rows of whole 256-element groups: Adam runs inside the projection kernel, so the
    # workspace holds N~ (bf16 r x n) and P~ (bf16 m x r) but no fp32 R
    assert B.lib().qgalore_workspace_bytes(256, 256, 32) >= 32 * 256 * 2 + 256 * 32 * 2
    assert B.lib().qgalore_workspace_bytes(4096, 4096, 1024) >= 4096 * 1024 * 4
    # ragged rows (n % 256 != 0): the fp32 partial sums of R are kept as well
    assert B.lib().qgalore_workspace_bytes(256, 200, 32) >= 32 * 200 * (4 + 2) + 256 * 32 * 2
    assert B.lib().qgalore_workspace_bytes(256, 256, 12) == 0
    assert B.lib().qgalore_cossim_workspace_bytes(4096, 128) >= 5 * 128 * 128 * 4
    assert B.lib().qgalore_cossim_workspace_bytes(100, 128) == 0


def test_refresh_workspace_size_query():
    """Sketch widths up to 2048 (the wide path above 136: fp64 block Jacobi buffers and the
    fp32 products' partial sums) and gradients whose column count is not a multiple of 8 (a
    zero-padded copy of G)."""
    q = B.lib().qgalore_refresh_workspace_bytes
    small = q(4096, 4096, 128, 8)
    assert small >= 3 * 4096 * 136 * 4
    wide = q(4096, 4096, 1024, 8)
    K = 1088   # 1032 padded to an even number of 32-index blocks
    assert wide >= 3 * 4096 * 1032 * 4 + 2 * K * K * 8
    ragged = q(2048, 5461, 512, 8)
    assert ragged >= 2048 * 5464 * 2 + 3 * 5461 * 520 * 4
    assert q(4096, 4096, 2040, 8) > 0          # k = 2048, the widest sketch
    assert q(4096, 4096, 2048, 8) == 0         # k = 2056
    assert q(1000, 1040, 1024, 24) == 0        # k = 1048 > m
    assert q(512, 389, 32, 8) > 0              # n % 8 != 0 is accepted


def test_other_entry_points_validate_first():
    L = B.lib()
    p = B.Proj(m=256, r=32, q=0x10000, scale=0x10000)
    bad = B.Proj(m=256, r=32, q=None, scale=0x10000)
    out = ctypes.c_float()
    assert L.qgalore_cossim(ctypes.byref(bad), ctypes.byref(p), 0x10000, 1 << 30, None,
                            ctypes.byref(out)) == 1
    q2 = B.Proj(m=128, r=32, q=0x10000, scale=0x10000)
    assert L.qgalore_cossim(ctypes.byref(q2), ctypes.byref(p), 0x10000, 1 << 30, None,
                            ctypes.byref(out)) == 2
    assert L.qgalore_cossim(ctypes.byref(p), ctypes.byref(p), 0x10000, 16, None,
                            ctypes.byref(out)) == 4
    assert L.qgalore_quantize_proj(None, 4, 4, 0x10000, 0x10000, None) == 1
    assert L.qgalore_quantize_proj(0x10004, 4, 4, 0x10000, 0x10000, None) == 3
    handle = ctypes.c_void_p()
    assert L.qgalore_plan_create(None, 1, ctypes.byref(handle)) == 1
    arr = (B.Layer * 2)()
    for k in range(2):
        arr[k].desc = _desc()
        for f in ("G", "W_q", "W_scale", "P_q", "P_scale", "M_q", "V_q"):
            setattr(arr[k], f, 0x10000)
    arr[1].desc.beta2 = 0.99
    assert L.qgalore_plan_create(arr, 2, ctypes.byref(handle)) == 5   # betas must agree
    assert L.qgalore_plan_step(None, 1, 0, 0x10000, 1, None) == 1


def test_valid_arguments_without_a_gpu_report_no_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _call(_desc()) == 7


def test_library_schedule_matches_oracle_schedule():
    """The host-side schedule in the library against the oracle's, on random similarity
    sequences with values at, above and below the threshold."""
    rng = np.random.default_rng(5)
    for trial in range(50):
        delta0 = int(rng.integers(1, 40))
        T = int(rng.integers(50, 400))
        vals = rng.choice([0.1, 0.39999, 0.4, 0.40001, 0.9], size=T)
        lib_s = B.Schedule(delta0, 0.4)
        ora = O.LayerSchedule(delta=delta0, gamma=np.float32(0.4))
        for t in range(T):
            assert lib_s.due(t) == ora.due(t)
            if ora.due(t):
                cs = float(np.float32(vals[t]))
                assert lib_s.refresh(t, cs if ora.count else None) == ora.refresh(t, cs if ora.count else None)
                assert (lib_s.delta, lib_s.next_refresh, lib_s.count) == (ora.delta, ora.next_refresh, ora.count)


def test_mfma_probe_rejects_bad_arguments_before_hip():
    L = B.lib()
    buf = (ctypes.c_uint16 * 64)()
    out = (ctypes.c_float * 256)()
    p = ctypes.cast(buf, ctypes.c_void_p)
    o = ctypes.cast(out, ctypes.c_void_p)
    assert L.qgalore_mfma_probe(None, 64, o, 1, 1, None) == 1            # QG_ERR_NULL
    assert L.qgalore_mfma_probe(p, 60, o, 1, 1, None) == 2               # not a multiple of 8
    assert L.qgalore_mfma_probe(p, 0, o, 1, 1, None) == 2
    assert L.qgalore_mfma_probe(p, 64, o, 0, 1, None) == 5               # grid < 1
    assert L.qgalore_mfma_probe(p, 64, o, 1, 0, None) == 5               # iters < 1
    assert L.qgalore_mfma_probe(p, 64, o, 70000, 1, None) == 5


def test_plan_projection_cache_entry_points_reject_null():
    L = B.lib()
    assert L.qgalore_plan_cache_proj(None, 1) == 1            # QG_ERR_NULL
    assert L.qgalore_plan_proj_changed(None, 0) == 1
