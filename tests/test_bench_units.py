"""The benchmark's algorithmic work units, checked against figures worked out from
the block's shapes (xserv "Phase 19: gpt-oss-20b MoE support", section 1:
hidden 2880, expert intermediate 2880, top-4; 32 or 128 experts) and written
down before the benchmark code existed:

* a live bf16 expert is 49,766,400 bytes of weights (gate_up 33,177,600, down
  16,588,800) plus 17,280 bytes of biases;
* one token costs 199.25 MFLOP at E = 32 and 199.80 MFLOP at E = 128 (router,
  gate_up and down; the GLU epilogue is not counted);
* per batch: c2 (T = 64, all 32 experts live) moves 1.594 GB and 12.75 GFLOP,
  c3 (T = 4096) 1.640 GB and 816.1 GFLOP, c5 (T = 16384, all 128 experts live)
  6.562 GB and 3273.6 GFLOP;
* the gate_up launch at c3 is 543.6 GFLOP;
* an MXFP4 expert's gate_up weight is 8.81 MB and its down weight 4.41 MB (half
  a byte per value, one scale byte per 32); an FP8 expert's are 16.59 MB and
  8.29 MB (one byte per value and one float32 scale).

CPU only: nothing here touches a GPU.
"""
from __future__ import annotations

import math
import os
import re

import pytest

import bench
from moe_layer_route_amd import datagen as d

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def close(value, expected, digits):
    """value rounds to the printed figure `expected` (given to `digits` significant digits)."""
    scale = 10 ** (math.floor(math.log10(abs(expected))) - digits + 1)
    return abs(value - expected) <= 0.5 * scale


def test_bf16_expert_bytes():
    cfg = d.CONFIGS["c2"]
    fixed = cfg.E * cfg.H * 2 + cfg.E * 2 + 2 * cfg.T * cfg.H * 2
    assert bench._alg_bytes_layer(cfg, 1) - fixed == 49_766_400 + 17_280
    gate_up_one = bench._alg_bytes_gate_up(cfg, 1) - bench._alg_bytes_gate_up(cfg, 0)
    assert gate_up_one == 33_177_600 + 11_520


@pytest.mark.parametrize("name,D,gbytes,gflops", [
    ("c2", 32, 1.594, 12.75),
    ("c3", 32, 1.640, 816.1),
    ("c5", 128, 6.562, 3273.6),
])
def test_layer_units(name, D, gbytes, gflops):
    cfg = d.CONFIGS[name]
    assert close(bench._alg_bytes_layer(cfg, D) / 1e9, gbytes, 4)
    assert close(bench._alg_flops_layer(cfg) / 1e9, gflops, 4)


@pytest.mark.parametrize("name,mflop", [("c2", 199.25), ("c5", 199.80)])
def test_flops_per_token(name, mflop):
    cfg = d.CONFIGS[name]
    assert close(bench._alg_flops_layer(cfg) / cfg.T / 1e6, mflop, 5)


def test_gate_up_flops_at_c3():
    cfg = d.CONFIGS["c3"]
    # the benchmark prices the gate_up launch at 2 T k H 2I flops
    src = open(os.path.join(ROOT, "bench.py")).read()
    assert re.search(r"gu_flops = 2 \* T \* k \* H \* 2 \* I\b", src)
    assert close(2 * cfg.T * cfg.k * cfg.H * 2 * cfg.I / 1e9, 543.6, 4)


def test_quantised_expert_bytes():
    H = I = 2880
    assert close(bench._mx_bytes(H, 2 * I) / 1e6, 8.81, 3)
    assert close(bench._mx_bytes(I, H) / 1e6, 4.41, 3)
    assert close(bench._f8_bytes(H, 2 * I) / 1e6, 16.59, 4)
    assert close(bench._f8_bytes(I, H) / 1e6, 8.29, 3)


def test_counter_summaries_parse():
    """Every committed HBM counter summary names its kernel, carries a source
    digest and a positive byte count, and its ratio to the algorithmic bytes
    matches the two figures it states."""
    prof = os.path.join(ROOT, "profiles")
    files = sorted(f for f in os.listdir(prof) if f.startswith("counters_") and f.endswith(".txt"))
    assert files
    for f in files:
        kv = {}
        for line in open(os.path.join(prof, f)):
            if "=" in line and not line.startswith("#"):
                a, b = line.split("=", 1)
                kv[a.strip()] = b.strip()
        assert kv.get("kernel"), f
        assert re.fullmatch(r"[0-9a-f]{16}", kv.get("source_digest", "")), f
        hbm = float(kv["hbm_bytes_per_launch"])
        alg = float(kv["alg_bytes_per_launch"])
        assert hbm > 0 and alg > 0, f
        assert abs(hbm / alg - float(kv["traffic_over_alg"])) < 1e-3, f
