"""Host logic of bench.py, on the CPU: the algorithmic byte and FLOP
accounting, the guard that drops stale traffic counters, the packing report,
and the one-GPU refusal."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
from oracle import pack_plan as ref_plan


def test_algorithmic_bytes_per_token():
    """Each operator reads its inputs once and writes its outputs once
    (bf16 (T, D) tensors, bf16 B/C rows, fp32 dB/dC rows, int32 positions):
    at d_inner 4096, d_state 16 a token moves 16 388 B through the conv
    forward, 32 836 B through the scan forward, 57 540 B through the scan
    backward and 24 580 B through the conv backward."""
    b = bench.algo_bytes(1, 4096, 16)
    assert b["conv_fwd"] == 4096 * (2 + 2) + 4
    assert b["scan_fwd"] == 4096 * (2 * 3 + 2) + 16 * 2 * 2 + 4
    assert b["scan_bwd"] == 4096 * (2 * 4 + 2 * 3) + 16 * 2 * 2 + 16 * 2 * 4 + 4
    assert b["conv_bwd"] == 4096 * (2 * 2 + 2) + 4
    assert (b["conv_fwd"], b["scan_fwd"], b["scan_bwd"], b["conv_bwd"]) == (16388, 32836, 57540, 24580)
    assert b["conv_fwd"] + b["scan_fwd"] == 49224
    assert b["scan_bwd"] + b["conv_bwd"] == 82120
    # linear in tokens; fp32 doubles the element bytes only
    b2 = bench.algo_bytes(1000, 4096, 16)
    assert all(b2[k] == 1000 * b[k] for k in b)
    f = bench.algo_bytes(1, 8, 4, elt=4)
    assert f["conv_fwd"] == 8 * 8 + 4


def test_backward_flop_count():
    """The scan backward's own FLOPs per (t, d, n), FMA = 2, without the forward
    recompute: dh 2, dB and dC products with their channel sums 4, sum dh*B 2,
    r 2, sum A*r 2, dA 2, carry 1; priced against the fp32 vector peak without
    packed FP32 (256 CUs x 4 SIMD16 x 2 FLOP x 2.4 GHz)."""
    assert bench.SCAN_BWD_FLOPS_PER_TDN == 2 + 4 + 2 + 2 + 2 + 2 + 1
    assert abs(bench.PEAK_FP32_TFLOPS - 256 * 4 * 16 * 2 * 2.4e9 / 1e12) < 0.1


def test_traffic_reported_only_for_the_measured_sources(monkeypatch):
    """Counter bytes are reported while the kernel sources hash to the value
    they were taken on, and null otherwise (or for an operator never measured)."""
    m = bench.MEASURED_TRAFFIC["scan_bwd"]
    current = bench.source_digest(m["sources"])
    monkeypatch.setitem(bench.MEASURED_TRAFFIC, "scan_bwd", dict(m, sha256=current))
    assert bench.measured_traffic("scan_bwd") == m["bytes"]
    monkeypatch.setitem(bench.MEASURED_TRAFFIC, "scan_bwd", dict(m, sha256="0" * 64))
    assert bench.measured_traffic("scan_bwd") is None
    assert bench.measured_traffic("conv_fwd") is None


def test_packing_report_matches_the_reference_packer():
    pytest.importorskip("torch")
    rep = bench.packing_report(n_docs=400)
    assert set(rep) == {bench.synth.NAMES[w] for w in (1, 2, 3)}
    for w in (1, 2, 3):
        row = rep[bench.synth.NAMES[w]]
        cap = bench.synth.WORKLOADS[w].pack_len
        docs = bench.synth.document_lengths(w, 400, seed=100 + w)
        assert row["tokens"] == int(sum(docs)) and row["capacity"] == cap
        for name, strategy, window in bench.PACK_STRATEGIES:
            _, _, bounds, _, padding = ref_plan.plan(np.asarray(docs), cap, strategy, window or 400)
            n_packs = len(bounds) - 1
            assert row[name]["packs"] == n_packs, name
            assert row[name]["padding_rate"] == round(padding / (n_packs * cap), 5), name


def test_more_than_one_gpu_is_refused():
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=root)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]
