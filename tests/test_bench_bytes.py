"""Host-side checks of the numbers bench.py divides by (no GPU): the
algorithmic bytes of every workload, written out tensor by tensor, the
roofline arithmetic, and that counter records taken on another kernel source
are not used.  Workload tensors are meta tensors (shapes, no memory)."""
import importlib.util
import json
import os

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def meta(*shape):
    return torch.empty(shape, device="meta")


BF16, F32 = 2, 4


def test_gated_headline_bytes(bench):
    B, T, N = 16, 8192, 2048
    # read a and u, write s; s0 read and s_final written once per channel
    expect = (2 * B * T * N + B * T * N) * F32 + B * N * F32 + B * N * F32
    assert bench.elem_bytes(B, T, N) == expect == 3_221_487_616


def test_mamba2_bytes(bench):
    B, T, H, K, V = 8, 4096, 24, 128, 64
    d = {"q": meta(B, T, 1, K), "k": meta(B, T, 1, K), "v": meta(B, T, H, V), "g": meta(B, T, H),
         "k_scale": meta(B, T, H)}
    expect = (2 * B * T * K) * BF16 + B * T * H * V * BF16 + 2 * B * T * H * F32 \
        + B * T * H * V * F32 + B * H * K * V * F32
    assert bench.diag_bytes(d) == expect == 331_350_016


def test_gla_bytes(bench):
    B, T, H, K, V = 4, 4096, 4, 128, 128
    d = {"q": meta(B, T, H, K), "k": meta(B, T, H, K), "v": meta(B, T, H, V), "g": meta(B, T, H, K),
         "k_scale": None}
    expect = 2 * B * T * H * K * BF16 + B * T * H * V * BF16 + B * T * H * K * F32 \
        + B * T * H * V * F32 + B * H * K * V * F32
    assert bench.diag_bytes(d) == expect == 118_489_088


@pytest.mark.parametrize("K,out,total", [(128, F32, 170_393_600), (64, F32, 135_790_592), (128, BF16, 136_839_168)])
def test_deltanet_bytes(bench, K, out, total):
    B, T, H, V = 4, 4096, 8, 128
    d = {"q": meta(B, T, H, K), "k": meta(B, T, H, K), "v": meta(B, T, H, V), "beta": meta(B, T, H)}
    expect = 2 * B * T * H * K * BF16 + B * T * H * V * BF16 + B * T * H * F32 \
        + B * T * H * V * out + B * H * K * V * F32
    assert bench.delta_bytes(d, out) == expect == total


@pytest.mark.parametrize("H,K,total", [(12, 64, 177_733_632), (8, 128, 237_502_464)])
def test_decayed_delta_bytes(bench, H, K, total):
    B, T = 4, 4096
    V = K
    d = {"q": meta(B, T, H, K), "k": meta(B, T, H, K), "v": meta(B, T, H, V), "beta": meta(B, T, H),
         "g": meta(B, T, H, K)}
    expect = 2 * B * T * H * K * BF16 + B * T * H * V * BF16 + B * T * H * F32 + B * T * H * K * F32 \
        + B * T * H * V * F32 + B * H * K * V * F32
    assert bench.delta_bytes(d, F32) == expect == total


def test_roofline_arithmetic(bench):
    r = bench.roofline(4_000_000_000, 1.0, copy=5000.0)   # 4 GB in 1 ms
    assert r["achieved"] == 4000.0 and r["frac"] == 0.5 and r["peak"] == 8000.0
    assert r["bytes_per_call"] == 4_000_000_000 and r["frac_of_copy"] == 0.8 and r["bound"] == "hbm"


def test_counter_records_need_the_current_source(bench, tmp_path, monkeypatch):
    rec = {"k_now": {"source_sha": bench.source_sha("scan_elem.hip"), "bytes_per_launch": 123},
           "k_old": {"source_sha": "0" * 16, "bytes_per_launch": 456}}
    (tmp_path / "traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.measured_traffic("k_now", "scan_elem.hip") == 123
    assert bench.measured_traffic("k_old", "scan_elem.hip") is None
    assert bench.measured_traffic("k_missing", "scan_elem.hip") is None


def test_committed_records_match_the_sources(bench):
    # every record in profiles/traffic.json was taken on the kernel source now in the tree
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        recs = json.load(f)
    stale, checked = [], 0
    for key, rec in recs.items():
        if not isinstance(rec, dict) or "source_sha" not in rec:
            continue
        f = "scan_elem.hip" if "elem" in key else ("scan_diag_outer.hip" if key.startswith("diag") else "scan_delta.hip")
        checked += 1
        if rec["source_sha"] != bench.source_sha(f):
            stale.append(key)
    assert checked > 30 and not stale, (checked, stale)
