"""bench.py on the CPU: the one-GPU guard and the host-side helpers (no kernel runs)."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import oracle as O  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode != 0
    assert "one GPU" in res.stderr
    assert res.stdout.strip() == ""          # no JSON line for a refused run


def test_kept_tile_flops_matches_the_oracle_count():
    rng = np.random.default_rng(3)
    B, H, N, blk, d = 2, 3, 1000, 128, 64
    Nb = O.num_blocks(N, blk)
    M = rng.random((B, H, Nb, Nb)) < 0.3
    rp, ci = O.to_csr(M)
    assert bench.kept_tile_flops(rp, ci, N, blk, d, H, B) == O.kept_tile_flops(M, N, blk, d)


def test_traffic_record_is_ignored_when_the_sources_change(tmp_path, monkeypatch):
    import json
    import hashlib
    rec = json.load(open(os.path.join(ROOT, "profiles", "attn_fwd_wan_traffic.json")))
    # the sources under another root, with a record made for them: reported while the hash
    # matches, not after a change
    h = hashlib.sha256()
    for rel in rec["sources"]:
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        data = open(os.path.join(ROOT, rel), "rb").read()
        dst.write_bytes(data)
        h.update(data)
    rec["source_sha256"] = h.hexdigest()
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "attn_fwd_wan_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.load_traffic("attn_fwd_wan") == rec["bytes_per_launch"]
    with open(tmp_path / rec["sources"][0], "ab") as f:
        f.write(b"\n// edited\n")
    assert bench.load_traffic("attn_fwd_wan") is None
