"""Host-side logic of bench.py (no GPU): the per-call HBM counter summary, the
mapping of the step's calls to the standalone calls the counters are taken on,
the digest check that voids stale counter bytes, the algorithmic byte counts, and
the refusal of a multi-GPU run."""
import csv
import dataclasses
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from mtp_draft_verification_amd import configs  # noqa: E402


def _write_counters(d, rows):
    """rows: (dispatch id, kernel name, counter, value in KiB) as rocprofv3's csv has them."""
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, name, ctr, v in rows:
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": ctr, "Counter_Value": v})


def test_pmc_summary_per_call_bytes_and_copy_scaling(tmp_path):
    fetch, write = tmp_path / "fetch", tmp_path / "write"
    copy = "void at::native::copy_kernel"
    gib_kib = (1 << 30) / 1024
    # the 1 GiB copy: FETCH reads half the bytes read (factor 2), WRITE all of them (factor 1)
    for root, ctr, v in ((fetch, "FETCH_SIZE", gib_kib / 2), (write, "WRITE_SIZE", gib_kib)):
        _write_counters(root / "hbm_copy", [(i, copy, ctr, v) for i in range(6)] +
                        [(9, "void sv::fill(int)", ctr, 1.0)])
    # a call of two library kernels made 3 times, plus a torch kernel that must not count
    att, mrg = "void sv::attn_mfma_kernel<512, 2, true, false>(sv::AttnParams)", "sv::attn_merge_kernel(sv::AttnParams)"
    rows_f, rows_w = [], []
    for c in range(3):
        rows_f += [(10 * c, att, "FETCH_SIZE", 1000.0), (10 * c + 1, mrg, "FETCH_SIZE", 10.0),
                   (10 * c + 2, "void at::native::fill", "FETCH_SIZE", 5000.0)]
        rows_w += [(10 * c, att, "WRITE_SIZE", 20.0), (10 * c + 1, mrg, "WRITE_SIZE", 4.0)]
    # a one-time setup kernel of the library (weight tiling) is not part of the call
    rows_f.append((99, "sv::tile_weights_kernel(unsigned short const*, unsigned short*, int, int, int, int, long)",
                   "FETCH_SIZE", 9000.0))
    _write_counters(fetch / "attn_global", rows_f)
    _write_counters(write / "attn_global", rows_w)
    with open(fetch / "attn_global.json", "w") as f:
        f.write(json.dumps({"call": "attn_global", "alg_bytes": 2_000_000}) + "\n")
    out = bench.pmc_summary([str(fetch), str(write)], out_path=str(tmp_path / "t.json"))
    assert out["copy_scale"] == {"FETCH_SIZE": 2.0, "WRITE_SIZE": 1.0}
    e = out["calls"]["attn_global"]
    assert e["calls_counted"] == 3
    assert e["FETCH_SIZE_KiB_per_call_raw"] == 1010.0 and e["WRITE_SIZE_KiB_per_call_raw"] == 24.0
    assert e["bytes_per_call"] == round((1010.0 * 2 + 24.0) * 1024)
    assert e["traffic_over_alg"] == round(e["bytes_per_call"] / 2_000_000, 4)
    assert json.load(open(tmp_path / "t.json"))["calls"]["attn_global"] == e


def test_step_calls_map_to_their_standalone_calls():
    cfg = configs.STACK
    kinds = [ly.window == 0 for ly in cfg.layers]
    assert bench.only_call(cfg, "lmhead") == "lmhead"
    for i, is_global in enumerate(kinds):
        kind = "global" if is_global else "local"
        assert bench.only_call(cfg, f"L{i}.attn") == f"attn_{kind}"
        assert bench.only_call(cfg, f"L{i}.qkv") == f"qkv_{kind}"
        assert bench.only_call(cfg, f"L{i}.o") == f"o_{kind}"
        assert bench.only_call(cfg, f"L{i}.gu") == "gu" and bench.only_call(cfg, f"L{i}.down") == "down"
    assert bench.only_call(cfg, "embed") is None and bench.only_call(cfg, "final_norm") is None


def test_traffic_is_void_unless_taken_on_the_current_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    body = {"calls": {"lmhead": {"bytes_per_call": 123}}}
    (prof / "hbm_traffic.json").write_text(json.dumps({**body, "source_digest": "not-these-sources"}))
    assert bench.load_traffic("lmhead") is None
    (prof / "hbm_traffic.json").write_text(json.dumps({**body, "source_digest": bench.source_digest()}))
    assert bench.load_traffic("lmhead") == 123.0
    assert bench.load_traffic("gu") is None and bench.load_traffic(None) is None


def test_algorithmic_bytes_of_the_step():
    cfg = dataclasses.replace(configs.STACK, batch=8, k=4)
    L = 131072
    cb = bench.call_bytes(cfg, [L] * 8)
    R, d, V = 40, cfg.d_model, cfg.vocab
    assert cb["lmhead"] == V * d * 2 + R * d * 2
    glo = cfg.layers[-1]
    keys = 8 * (L + cfg.k + 1) * glo.n_heads_kv
    assert cb["L5.attn"] >= keys * glo.head_dim * 2          # K = V: the key tile read once
    loc = cfg.layers[0]
    assert cb["L0.attn"] < cb["L5.attn"] / 10                  # the window caps the local read
    assert cb["L0.gu"] >= 2 * cfg.d_ff * d * 2 and cb["L0.down"] >= cfg.d_ff * d * 2
    assert cb["L0.qkv"] >= (loc.n_heads_q + 2 * loc.n_heads_kv) * loc.head_dim * d * 2


def test_multi_gpu_run_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
