"""bench.py's parts that hold without a GPU: it measures one GPU and refuses a
multi-GPU request (an argument or a launcher's WORLD_SIZE) with a message and
exit status 2, before touching any device; the parity record of its JSON
line counts every difference between a run's outputs and the oracle's; and
its roofline traffic figure is the committed counter summary of the current
GEMM source, or null."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2", "--steps", "1", "--warmup", "0"])
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)
    assert r.stdout.strip() == "" or not r.stdout.strip().startswith("{")  # no JSON line


def test_a_launcher_world_size_above_one_is_refused():
    r = _run(["--steps", "1", "--warmup", "0"], {"WORLD_SIZE": "2", "RANK": "0", "LOCAL_RANK": "0"})
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)


def _bench_module():
    import importlib.util

    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_parity_record_counts_planted_mismatches():
    """The JSON line's cpu_baseline.parity: the helper that compares a run's
    outputs with the oracle's counts every planted difference and reports the
    error of the 16-bit outputs."""
    import numpy as np

    import oracle.pdq_oracle as O
    from w8a8_int8_quantized_absmax_amd import synth

    b = _bench_module()
    t = synth.Tiny()
    x, w = t.x(), t.w()
    rq, rs, rc = O.quantize_weight(w)
    ref = O.linear_prefill(x, rq, rs)
    g = dict(xq=ref["xq"].copy(), x_scale=ref["x_scale"].copy(), acc=ref["acc"].copy(),
             y=O.to_bf16_bits(ref["y32"]))
    clean = b._parity(O, g, ref)
    assert clean["code_mismatches"] == clean["acc_mismatches"] == clean["y_bits_mismatches"] == 0
    assert clean["scale_mismatches"] == 0 and clean["y_mae"] == 0.0 and clean["y_max_rel_err"] < 4e-3
    g["xq"][0, 0] ^= 1
    g["acc"][1, 2] += 1
    g["acc"][3, 4] -= 1
    g["x_scale"][5] = np.nextafter(g["x_scale"][5], np.float32(2))
    g["y"][2, 2] ^= 0x40
    bad = b._parity(O, g, ref)
    assert (bad["code_mismatches"], bad["acc_mismatches"], bad["scale_mismatches"], bad["y_bits_mismatches"]) == \
        (1, 2, 1, 1)
    assert bad["y_mae"] > 0.0

    d = O.linear_decode(x, np.float32(0.5), 3, rq, rs, rc)
    gd = dict(xq=d["xq"].copy(), acc=d["acc"].copy(), y=O.to_bf16_bits(d["y32"]), sat=d["sat"] + 1)
    assert b._parity(O, gd, d)["saturation_count_equal"] is False

    x8 = synth.round_to(x, "f16")
    w8 = synth.round_to(w, "f16")
    q8, s8, _ = O.quantize_weight(w8)
    r8 = O.linear_int8_outlier(x8, w8, q8, s8, 6.0)
    g8 = dict(idx=r8["cols"].astype(np.int32), count=len(r8["cols"]), xq=r8["xq"].copy(),
              x_scale=r8["x_scale"].copy(), acc=r8["acc"].copy(), y=O.to_f16(r8["y64"]).view(np.uint16).copy())
    ok8 = b._parity_llm_int8(O, g8, r8)
    assert ok8["outlier_columns_equal"] and ok8["acc_mismatches"] == 0 and ok8["y_mae"] == 0.0
    g8["count"] += 1
    g8["acc"][0, 0] += 7
    bad8 = b._parity_llm_int8(O, g8, r8)
    assert not bad8["outlier_columns_equal"] and bad8["acc_mismatches"] == 1


def test_traffic_summary_is_for_the_current_gemm_and_adds_up(tmp_path):
    """roofline.traffic comes from the committed counter summary only while it
    was taken on the current GEMM source: its bytes are the two counters scaled
    by the copy-kernel calibration, and any code change to the GEMM source (not
    a comment) makes the bench line report null instead."""
    import json

    b = _bench_module()
    with open(b.TRAFFIC_FILE) as f:
        t = json.load(f)
    cal = t["calibration"]
    # a 1 GiB copy reads and writes 1 GiB: the scales follow from its counters
    assert cal["fetch_scale"] == round(1048576.0 / cal["copy_FETCH_SIZE_KiB"], 2)
    assert cal["write_scale"] == round(1048576.0 / cal["copy_WRITE_SIZE_KiB"], 2)
    fetch = t["FETCH_SIZE_KiB_per_launch"] * 1024 * cal["fetch_scale"]
    write = t["WRITE_SIZE_KiB_per_launch"] * 1024 * cal["write_scale"]
    assert (fetch, write) == (t["fetch_bytes_per_launch"], t["write_bytes_per_launch"])
    assert t["bytes_per_launch"] == fetch + write
    # the written bytes are the bf16 output of the 4096 x 11008 product
    assert t["write_bytes_per_launch"] == 4096 * 11008 * 2
    assert t["bytes_per_launch"] >= t["algorithmic_bytes_per_launch"]
    assert b.traffic_for(0) == t["bytes_per_launch"], "counters were taken on another GEMM source"

    with open(b.GEMM_SRC) as f:
        src = f.read()
    edited = tmp_path / "gemm_i8.hip"
    edited.write_text(src + "\n// a comment only\n")
    b.GEMM_SRC = str(edited)
    assert b.traffic_for(0) == t["bytes_per_launch"]
    edited.write_text(src + "\nstatic int unused_probe;\n")
    assert b.traffic_for(0) is None
