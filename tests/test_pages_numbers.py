"""Host-side counting helpers against the numbers the pages print (CPU only)."""
import json
import os

import pytest
import torch

import workloads as W
from parity import TOL

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))


def test_attention_flop_count_matches_eq_f_share():
    g = GOLD["flop_share"]
    B, S, d, f = g["B"], g["S"], g["d_model"], g["ffn_mult"] * g["d_model"]
    H = 8
    w = W.Workload("eqf", B, H, S, S, d // H, False, ("f32",))
    attn = w.flops()                         # 4*B*H*S_q*S_kv*D = 4BS^2d
    total = 8 * B * S * d * d + attn + 4 * B * S * d * f
    share = 100.0 * attn / total
    assert round(share, 1) == g["attention_share_percent"]
    assert round(1.0 / (1.0 - g["attention_share_percent"] / 100), 3) == g["amdahl_bound"]
    wc = W.Workload("eqf_causal", B, H, S, S, d // H, True, ("f32",))
    assert wc.flops() == attn / 2


def test_case14_memory_sizes_pin_head_shape():
    g = GOLD["case14_memory"]
    B, S = g["batch"], g["seq_len"]
    H, D = 16, 64                      # d_model 1024 split in 16 heads of 64
    q_bytes = B * H * S * D * 4         # fp32 Q
    scores = B * H * S * S * 4          # fp32 [B,H,S,S]
    assert round(q_bytes / 1e9) == g["q_gb_approx"]
    assert round(scores / 1e12) == g["scores_tb_approx"]
    w = W.Workload("case14", B, H, S, S, D, False, ("f32",))
    assert w.bytes("f32") == 4 * q_bytes    # Q, K, V read and O written once


def _ulp(x, dtype):
    t = torch.tensor([x], dtype=dtype)
    nxt = torch.nextafter(t, torch.tensor([float("inf")], dtype=dtype))
    return float(nxt.float() - t.float())


def test_bf16_and_fp16_ulp_arithmetic():
    g = GOLD["bf16_ulp"]
    u = _ulp(g["magnitude"], torch.bfloat16)
    assert u == g["ulp"]
    assert round(100 * g["error"] / g["magnitude"], 2) == g["relative_percent"]
    assert round(0.01 * g["magnitude"] / u, 3) == g["tolerance_ulp"]
    h = GOLD["fp16_ulp"]
    uh = _ulp(h["magnitude"], torch.float16)
    assert round(100 * 2 * uh / h["magnitude"], 2) == h["relative_percent_2ulp"]


def test_fp32_tolerance_is_the_strict_published_pair():
    g = GOLD["tolerances"]["strict"]
    assert TOL["f32"] == (g["atol"], g["rtol"])


def test_ridge_point_arithmetic():
    g = GOLD["roofline_ridge"]
    assert round(g["tflops"] * 1e12 / (g["gbps"] * 1e9), 1) == g["ridge_flop_per_byte"]
