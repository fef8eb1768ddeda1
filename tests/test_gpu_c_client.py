"""The C ABI from plain C: tests/c_client/pdq_c_client (built by build()) runs the
weight quantization, the static calibration, the prefill linear and the decode
linear through libpdq's entry points on hipMalloc'd memory, with no Python
or PyTorch in the process; its outputs must equal the oracle's bit for bit
(codes, scales, column sums, calibration state, S and Z, accumulators,
saturation count, and the bf16 outputs, whose binary32 operation sequence
both sides share).  The tiny linear workload (X f32 [16, 256] with channels 3
and 77 x50, W f32 [512, 256], its 8 calibration batches stacked into one: the
MinMax state is order-free) and two larger shapes, one per GEMM kernel."""
import os
import subprocess

import numpy as np
import pytest

import oracle.pdq_oracle as O
from w8a8_int8_quantized_absmax_amd import pdq, synth
from packing import pack, pack_weight

pytestmark = pytest.mark.gpu

CLIENT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_client", "pdq_c_client")


def _cases():
    t = synth.Tiny()
    yield "tiny", t.x(), t.w(), np.concatenate([t.calib(b) for b in range(t.n_calib)])
    for m, n, k in ((300, 700, 1040), (2048, 2600, 512)):
        x = synth.activations(9800 + m, m, k, [1, k - 2], 100.0, offset=0.1, dtype="f32")
        w = synth.weights(9900 + n, n, k, "f32")
        cal = synth.activations(9950 + m, 64, k, [1, k - 2], 100.0, offset=0.1, dtype="f32")
        yield f"{m}x{n}x{k}", x, w, cal


@pytest.mark.parametrize("case", list(range(3)))
def test_c_client_matches_oracle(case, tmp_path):
    assert os.path.exists(CLIENT), "the C client is not built: run __graft_entry__.build()"
    name, x, w, cal = list(_cases())[case]
    m, k = x.shape
    n = w.shape[0]
    inp, outp = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(np.array([m, n, k, cal.shape[0]], np.int64).tobytes())
        for a in (x, w, cal):
            f.write(np.ascontiguousarray(a, np.float32).tobytes())
    print(f"C client case {name}: M={m} N={n} K={k}", flush=True)
    res = subprocess.run([CLIENT, str(inp), str(outp)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    raw = np.fromfile(outp, np.uint8)
    off = 0

    def take(count, dt):
        nonlocal off
        nb = count * np.dtype(dt).itemsize
        a = raw[off:off + nb].view(dt)
        off += nb
        return a

    wb, ab = pdq.weight_bytes(n, k), pdq.act_bytes(m, k)
    wq, ws, cs = take(wb, np.int8), take(n, np.float32), take(n, np.int32)
    xq, xs, y, acc = take(ab, np.int8), take(m, np.float32), take(m * n, np.uint16), take(m * n, np.int32)
    mm, s, z = take(2, np.float32), take(1, np.float32), take(1, np.int32)
    xq_d, y_d, acc_d, sat = take(ab, np.int8), take(m * n, np.uint16), take(m * n, np.int32), take(1, np.uint32)
    assert off == raw.size

    rq, rs, rc = O.quantize_weight(w)
    assert np.array_equal(wq, pack_weight(rq))
    assert np.array_equal(ws.view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(cs, rc)

    ref = O.linear_prefill(x, rq, rs)
    assert np.array_equal(xq, pack(ref["xq"]))
    assert np.array_equal(xs.view(np.uint32), ref["x_scale"].view(np.uint32))
    assert np.array_equal(acc.reshape(m, n), ref["acc"])
    assert np.array_equal(y.reshape(m, n), O.to_bf16_bits(ref["y32"]))

    state, rs_a, rz_a = O.calibrate([cal])
    assert np.array_equal(mm, np.array(state, np.float32))
    assert s.view(np.uint32)[0] == np.array([rs_a], np.float32).view(np.uint32)[0] and int(z[0]) == rz_a

    dref = O.linear_decode(x, rs_a, rz_a, rq, rs, rc)
    assert np.array_equal(xq_d, pack(dref["xq"]))
    assert int(sat[0]) == dref["sat"]
    assert np.array_equal(acc_d.reshape(m, n), dref["acc"])
    assert np.array_equal(y_d.reshape(m, n), O.to_bf16_bits(dref["y32"]))
