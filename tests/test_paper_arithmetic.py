"""The shapes this build assumes reproduce the figures the pages print
(tests/golden/paper_figures.json, each entry cited), and the cycle
arithmetic used for reporting reproduces the pages' worked example."""

import json
import os

import pytest

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "paper_figures.json")))

D, V, L, HQ, HKV, HD, INTER = 2560, 262144, 5, 32, 8, 128, 5120
MiB, GiB = 2 ** 20, 2 ** 30


def draft_parameter_count():
    head = V * D
    wc = 5 * D * D
    per_layer = (D * HQ * HD + 2 * D * HKV * HD + HQ * HD * D
                 + 3 * D * INTER + 2 * D + 2 * HD)
    return head, wc + head + L * per_layer + 2 * D


def test_parameter_count_and_head_share():
    head, total = draft_parameter_count()
    assert total == GOLD["draft_parameters"]["value"]
    assert round(100 * head / total, 1) == GOLD["head_share_percent"]["value"]
    assert round(total * 0.5 / MiB, 1) == GOLD["all_codes_4bit_MiB"]["value"]
    assert head * 0.5 / MiB == GOLD["head_codes_4bit_MiB"]["value"]
    assert V * D * 2 / GiB == GOLD["embedding_bf16_GiB"]["value"]


def test_cache_payload():
    per_seq = L * HKV * 1024 * HD * 2 * 2  # K and V, bf16
    assert per_seq / MiB == GOLD["cache_payload_per_seq_MiB"]["value"]
    assert 64 * per_seq / GiB == GOLD["cache_payload_64_seq_GiB"]["value"]


def test_fusion_matrix_size():
    assert round(2048 * 5 * 2048 * 2 / 1e6, 2) == GOLD["wc_bf16_MB_at_D2048"]["value"]


def cycle_speedup(t_draft_ms, t_verify_ms, tau, baseline_tok_s):
    """Per-token latency (T_draft + T_verify) / tau, its throughput, and the
    speedup over the bandwidth-bound baseline (DFlash & DFlash2, section 2)."""
    per_token = (t_draft_ms + t_verify_ms) / tau
    thr = 1000.0 / per_token
    return per_token, thr, thr / baseline_tok_s


def test_worked_cycle_example():
    bw = GOLD["bandwidth_bound_tok_s"]
    base = bw["inputs"]["bandwidth_GB_s"] / bw["inputs"]["weights_GB"]
    assert round(base, 2) == bw["value"]
    w = GOLD["worked_cycle"]
    per_token, thr, sp = cycle_speedup(w["inputs"]["T_draft_ms"], w["inputs"]["T_verify_ms"],
                                       w["inputs"]["tau"], round(base, 2))
    assert round(per_token, 2) == w["per_token_ms"]
    # The page derives throughput from the rounded 16.22 ms and prints it
    # as "approximately 61.6" (1000 / 16.22 = 61.65).
    thr_page = 1000.0 / w["per_token_ms"]
    assert abs(thr_page - w["throughput_tok_s"]) < 0.06
    assert abs(thr - w["throughput_tok_s"]) < 0.07
    assert round(w["throughput_tok_s"] / bw["value"], 2) == w["speedup_x"]
    assert abs(sp - w["speedup_x"]) < 0.01
