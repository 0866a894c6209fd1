"""Host-side checks of bench.py (no GPU): the one-GPU contract, the
algorithmic byte count and the roofline record of the dominant launch."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from weight_only_int4_gemv_amd import inputs  # noqa: E402


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(args, env):
    """The layer is built and measured on one GPU: N > 1 exits with status 2
    and says so, before touching a device."""
    e = dict(os.environ, **env)
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, env=e,
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr and p.stdout == ""


def test_gemv_bytes_of_the_sweep():
    """Codes (N*K/2) + fp16 scales per 128 (N*K/64) + x (2K) + y (2N): the
    gate_up launch and the whole LLaMA-3-8B sweep (32 layers, q/k/v and
    gate/up concatenated along N) as the bench line reports them."""
    assert bench.gemv_bytes(28672, 4096) == 28672 * 4096 // 2 + 28672 * 32 * 2 + 8192 + 57344
    assert bench.gemv_bytes(28672, 4096) == 60620800
    dims = {n: (K, N) for n, K, N in inputs.LLAMA3_8B}
    groups = bench.fused_groups([n for n, _, _ in inputs.LLAMA3_8B])
    per_layer = sum(bench.gemv_bytes(sum(dims[n][1] for n in g), dims[g[0]][0]) for g in groups)
    assert len(groups) == 4
    assert per_layer * inputs.LLAMA3_8B_LAYERS == 3603169280
    # M rows of X and Y scale the activation and output terms only
    assert bench.gemv_bytes(4096, 14336, M=16) - bench.gemv_bytes(4096, 14336) == \
        15 * 2 * (14336 + 4096)


def test_dominant_roofline_record(tmp_path, monkeypatch):
    """The launch with the largest time is chosen; achieved = its algorithmic
    bytes over its time; traffic only while the stored counter record matches
    the current GEMV sources."""
    layer0 = [(g, K, N, None, None, None) for g, K, N in
              [("q_k_v", 4096, 6144), ("o", 4096, 4096), ("gate_up", 4096, 28672),
               ("down", 14336, 4096)]]
    per_shape = {"q_k_v": {"K": 4096, "N": 6144, "us": 4.9},
                 "o": {"K": 4096, "N": 4096, "us": 4.3},
                 "gate_up": {"K": 4096, "N": 28672, "us": 12.5},
                 "down": {"K": 14336, "N": 4096, "us": 7.9}}
    rec = {"sources_sha256": bench.gemv_sources_sha256(),
           "per_launch": {"4096x28672": {"traffic_bytes": 61000000}}}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "PMC_TRAFFIC", str(path))
    r = bench.dominant_roofline(per_shape, layer0, 3603169280, 128, 7.5)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["bytes_per_launch"] == 60620800 and "gate_up" in r["kernel"]
    assert r["achieved"] == pytest.approx(60620800 / 12.5e-6 / 1e9, abs=0.05)
    assert r["frac"] == pytest.approx(r["achieved"] / 8000.0, abs=1e-4)
    assert r["traffic"] == 61000000
    rec["sources_sha256"] = "0" * 64
    path.write_text(json.dumps(rec))
    assert bench.dominant_roofline(per_shape, layer0, 3603169280, 128, 7.5)["traffic"] is None
    # without per-shape timings: the sweep's average launch, no traffic
    r = bench.dominant_roofline(None, layer0, 3603169280, 128, 7.5)
    assert r["traffic"] is None and r["bytes_per_launch"] == 3603169280 // 128
