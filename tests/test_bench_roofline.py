"""The roofline entry of bench.py picks the binding unit from the workload's algorithmic
counts: the largest of its lower-bound times on HBM (bytes / 8 TB/s), the bf16 matrix cores
(flops / 2516.6 TFLOP/s) and the vector ALUs (operations / 39.3 T lane operations per s)."""
import bench
from quantized_rank_gradient_amd import workloads as WL


def test_alu_peak_is_the_published_vector_peak_per_lane_operation():
    # 157.3 TFLOP/s fp32 vector = lane operations x 2 (an FMA) x 2 (packed fp32)
    assert abs(bench.ALU_PEAK_TOPS * 4 - 157.3) < 0.1


def test_rank_1024_back_projection_is_matrix_core_bound():
    cfg = WL.CONFIGS["llama7b_r1024"]
    rl = bench.roofline(cfg, cfg.r, (1.0, 14.0, 0.0, 15.0))
    assert rl["kernel"] == "qg_backproject" and rl["bound"] == "mfma"
    a = bench.algorithmic(cfg, cfg.r)
    assert abs(rl["achieved"] - a["flops"][3] / 15e-3 / 1e12) < 0.01


def test_rank_128_back_projection_is_alu_bound():
    """At rank 128 the product is 256 flops per weight and the rounding 13 operations: the
    vector ALUs bind before HBM (2 bytes per weight) and the matrix cores."""
    cfg = WL.CONFIGS["llama7b_r128"]
    rl = bench.roofline(cfg, cfg.r, (0.1, 2.8, 0.0, 4.7))
    assert rl["bound"] == "alu" and rl["unit"] == "TOP/s"
    lb = rl["lower_bound_ms"]
    assert lb["alu"] > lb["hbm"] > lb["mfma"]
    mn = sum(L.m * L.n for L in cfg.layers)
    assert abs(rl["achieved"] - bench.SR_OPS_PER_WEIGHT * mn / 4.7e-3 / 1e12) < 0.01


def test_rank_128_projection_alone_is_hbm_bound():
    """With the back-projection out of the way the projection binds on streaming G."""
    cfg = WL.CONFIGS["llama7b_r128"]
    rl = bench.roofline(cfg, cfg.r, (0.1, 2.8, 0.0, 0.0))
    assert rl["kernel"].startswith("qg_project") and rl["bound"] == "hbm"
