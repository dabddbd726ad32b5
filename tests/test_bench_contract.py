"""CPU checks of bench.py's contract that need no GPU: it refuses more than one GPU
before touching one, and its roofline `traffic` figure comes from the committed
counter record only while the kernel sources it was taken on are unchanged."""
import hashlib
import importlib.util
import json
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.pop("WORLD_SIZE", None)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          env=env, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run_bench(["--gpus", "2", "--steps", "1", "--warmup", "0"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_a_multi_rank_launch_is_refused():
    r = _run_bench(["--steps", "1", "--warmup", "0"], {"WORLD_SIZE": "2"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_follows_the_committed_record():
    """The committed figure while every recorded source hash matches the tree, else null."""
    bench = _bench_module()
    rec = json.load(open(os.path.join(ROOT, "profiles", "hbm_traffic.json")))
    current = all(
        hashlib.sha256(open(os.path.join(ROOT, "attention_shard_math_amd", "csrc", name), "rb").read()).hexdigest()
        == digest for name, digest in rec["source_sha256"].items())
    want = round(rec["kernels"]["mlp_col_gemm_gelu"]["hbm_bytes_per_launch"]) if current else None
    assert bench.traffic_from_profiles("mlp_col_gemm_gelu") == want
    assert bench.traffic_from_profiles("no_such_kernel") is None


def test_traffic_is_null_once_a_source_changes(tmp_path):
    # a copy of the record and its sources, the record's hashes taken from the copies;
    # then one source is edited
    (tmp_path / "profiles").mkdir()
    csrc = tmp_path / "attention_shard_math_amd" / "csrc"
    csrc.mkdir(parents=True)
    rec = json.load(open(os.path.join(ROOT, "profiles", "hbm_traffic.json")))
    for name in rec["source_sha256"]:
        shutil.copy(os.path.join(ROOT, "attention_shard_math_amd", "csrc", name), csrc / name)
        rec["source_sha256"][name] = hashlib.sha256((csrc / name).read_bytes()).hexdigest()
    (tmp_path / "profiles" / "hbm_traffic.json").write_text(json.dumps(rec))
    bench = _bench_module()
    bench.ROOT = str(tmp_path)
    assert bench.traffic_from_profiles("mlp_col_gemm_gelu") is not None
    first = sorted(rec["source_sha256"])[0]
    with open(csrc / first, "a") as f:
        f.write("\n// edited\n")
    assert bench.traffic_from_profiles("mlp_col_gemm_gelu") is None
