"""bench.py contract checks that need no GPU."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_traffic_summary_matches_kernel_or_is_dropped(tmp_path):
    sys.path.insert(0, ROOT)
    import bench
    tj = os.path.join(ROOT, "profiles", "ternary_gemv_traffic.json")
    v = bench.load_traffic(tj)
    assert v is None or v > 0
    bad = json.load(open(tj))
    bad["kernel_digest"] = "0" * 64
    p = tmp_path / "t.json"
    p.write_text(json.dumps(bad))
    assert bench.load_traffic(str(p)) is None


def test_traffic_digest_covers_only_the_kernel(tmp_path):
    """The digest changes with the measured kernel's body and not with an
    edit elsewhere in its source file."""
    sys.path.insert(0, ROOT)
    import bench
    src, spans, hdrs = bench.TRAFFIC_KERNEL
    text = open(os.path.join(ROOT, src)).read()
    base = bench.kernel_digest(src, spans, hdrs)
    rel = os.path.relpath(str(tmp_path / "k.hip"), ROOT)
    (tmp_path / "k.hip").write_text(text + "\n// appended\n")
    assert bench.kernel_digest(rel, spans, hdrs) == base
    body = text.replace("constexpr int kRowLds = CSW * 512;", "constexpr int kRowLds = CSW * 512 ;", 1)
    assert body != text
    (tmp_path / "k.hip").write_text(body)
    assert bench.kernel_digest(rel, spans, hdrs) != base


def test_algorithmic_bytes():
    sys.path.insert(0, ROOT)
    import bench
    # codes N*K/4 + fp16 scales + fp16 activations + fp16 outputs
    assert bench.ternary_bytes(1, 4096, 4096) == 4096 * 1024 + 2 * 4096 + 2 * 4096 + 2 * 4096


def test_sample_verdicts():
    """The CPU leg's parity check: an output equal to the oracle's product
    rounded to fp16 passes, one pushed past the bound fails, per line."""
    import numpy as np
    sys.path.insert(0, ROOT)
    import bench
    import oracle.gemm as OG
    import oracle.ternary as OT
    import synth
    W = synth.weights(32, 256, 5)
    codes, sb = OT.ternary_pack(W)
    A = synth.activations(2, 256, 6).double().numpy()
    out, mag = OG.gemm_ref64(A, OT.ternary_dequant(codes, sb, 256))
    good = out.astype(np.float16).astype(np.float64)
    bad = good.copy()
    bad[1, 3] += 2e-3 * mag[1, 3] + 2e-3
    smp = lambda line, C: {"line": line, "kind": "ternary", "K": 256, "dtype": "f16", "codes": codes,  # noqa: E731
                            "scale": sb, "A": A, "C": C}
    v = bench.check_samples([smp("a", good), smp("b", bad), smp("a", good)])
    assert v["lines"]["a"]["ok"] and v["lines"]["a"]["outputs"] == 2 * 2 * 32
    assert not v["lines"]["b"]["ok"] and not v["ok"]
