"""Host-side checks of bench.py (no GPU): every name its functions use is
defined, the one-GPU contract (--gpus N > 1 exits with a message), and the
counter-to-bytes arithmetic of the traffic summary on synthetic counter files."""
import ast
import builtins
import csv
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", BENCH)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_no_undefined_global_names():
    """A name loaded inside bench.py that is neither bound anywhere in the file
    nor a builtin would only fail at run time (on the GPU machine)."""
    tree = ast.parse(open(BENCH).read())
    bound = set(dir(builtins)) | {"__file__", "__name__", "__doc__"}
    for node in ast.walk(tree):
        if isinstance(node, (ast.FunctionDef, ast.ClassDef)):
            bound.add(node.name)
            if isinstance(node, ast.FunctionDef):
                for a in node.args.args + node.args.kwonlyargs:
                    bound.add(a.arg)
                if node.args.vararg:
                    bound.add(node.args.vararg.arg)
                if node.args.kwarg:
                    bound.add(node.args.kwarg.arg)
        elif isinstance(node, (ast.Import, ast.ImportFrom)):
            for a in node.names:
                bound.add((a.asname or a.name).split(".")[0])
        elif isinstance(node, ast.Name) and isinstance(node.ctx, (ast.Store, ast.Del)):
            bound.add(node.id)
        elif isinstance(node, ast.arg):
            bound.add(node.arg)
        elif isinstance(node, ast.ExceptHandler) and node.name:
            bound.add(node.name)
    used = {n.id for n in ast.walk(tree) if isinstance(n, ast.Name) and isinstance(n.ctx, ast.Load)}
    assert not (used - bound), f"bench.py uses undefined names: {sorted(used - bound)}"


def test_entry_functions_exist():
    b = load_bench()
    for name in ("cpu_baseline", "write_traffic", "measured_traffic", "bench_backward",
                 "calibration_copy", "traffic_paths", "kernels_digest", "main"):
        assert callable(getattr(b, name, None)), name


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True,
                       cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr


def test_traffic_from_counters(tmp_path, monkeypatch):
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch) scaled by the calibration
    copy's largest dispatch: a copy reading 0.5 GiB-equivalent of FETCH for
    1 GiB gives factor 2."""
    b = load_bench()
    out_json, out_txt = tmp_path / "t.json", tmp_path / "t.txt"
    monkeypatch.setattr(b, "traffic_paths", lambda backward, workload="block_L48_S8": (str(out_json), str(out_txt),
                                                              "attnres::phase2_kernel", ""))
    gib_kib = float(1 << 20)

    def write(path, counter, rows):
        with open(path, "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
            w.writeheader()
            for k, v in rows:
                w.writerow({"Kernel_Name": k, "Counter_Name": counter, "Counter_Value": v})

    fetch, wr = tmp_path / "f.csv", tmp_path / "w.csv"
    write(fetch, "FETCH_SIZE", [("__amd_rocclr_copyBuffer", gib_kib / 2), ("__amd_rocclr_copyBuffer", 3.0),
                                ("void attnres::phase2_kernel<a, 2, true, false>(P)", 100.0),
                                ("void attnres::phase2_kernel<a, 2, false, false>(P)", 60.0)])
    write(wr, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", gib_kib), ("__amd_rocclr_copyBuffer", 1.0),
                             ("void attnres::phase2_kernel<a, 2, true, false>(P)", 40.0),
                             ("void attnres::phase2_kernel<a, 2, false, false>(P)", 20.0)])
    t = b.write_traffic(str(fetch), str(wr), workload="w")
    assert abs(t["fetch_factor"] - 2.0) < 1e-12 and abs(t["write_factor"] - 1.0) < 1e-12
    # mean over the two variants' dispatches: ((100 * 2 + 40) + (60 * 2 + 20)) / 2 KiB
    assert abs(t["traffic_bytes_per_launch"] - 1024 * (240 + 140) / 2) < 1e-6
    assert json.load(open(out_json))["workload"] == "w"
