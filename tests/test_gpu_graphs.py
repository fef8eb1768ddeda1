"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: callers that cannot allocate or that replay graphs in a serving loop
capture them this way.  Each graph is replayed several times with new inputs
copied into its static input buffer by eager work between the replays, a
synchronisation after each replay, and an eager call of the same entry point
on the same input; every replay must give the eager call's outputs bit for
bit.  (The library enqueues no memset, copy or allocation, so a graph holds
only its kernels; a stale byte of one replay's scratch, counter or padding
that the next replay read would show here.)  The eager calls' parity with the
oracle is established by the other GPU tests."""
import numpy as np
import pytest
import torch

from w8a8_int8_quantized_absmax_amd import pdq, synth
from gpu_helpers import dev, host

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _bits(t):
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16)
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    return t


def _same(a, b, what):
    assert torch.equal(_bits(a), _bits(b)), what


def _replay_against_eager(call, x_static, inputs, compare):
    """Capture call(x_static), then for each input: copy it in, replay,
    synchronise, run call(input) eagerly and compare the two results."""
    call(x_static)  # eager warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        captured = call(x_static)
    for i, x in enumerate(inputs):
        x_static.copy_(x)
        g.replay()
        torch.cuda.synchronize()
        ref = call(x)
        torch.cuda.synchronize()
        compare(captured, ref, i)
    del g


def _x(seed, m, k, dtype="bf16", cols=(), mag=100.0):
    x = synth.normal(seed, (m, k))
    if cols:
        x[:, list(cols)] = synth.normal(seed + 1, (m, len(cols)), mag)
    return dev(synth.round_to(x, dtype), dtype)


@pytest.mark.parametrize("m", [1, 32])
def test_decode_call_in_a_graph(m):
    k, n = 4096, 1024
    wq, ws, cs = pdq.quantize_weight(dev(synth.weights(8100, n, k, "bf16"), "bf16"))
    s, z = np.float32(0.05), -3
    x_static = torch.empty((m, k), dtype=torch.bfloat16, device="cuda")
    inputs = [_x(8110 + i, m, k, cols=(7, 900)) for i in range(REPLAYS)]

    def call(x):
        return pdq.linear_decode(x, s, z, wq, ws, cs, want_acc=True)

    def compare(got, ref, i):
        _same(got["y"], ref["y"], f"y, replay {i}")
        _same(got["acc"], ref["acc"], f"acc, replay {i}")
        assert torch.equal(got["xq"].data, ref["xq"].data), f"codes, replay {i}"

    _replay_against_eager(call, x_static, inputs, compare)


@pytest.mark.parametrize("m,n,k", [(300, 640, 1024), (2048, 2048, 512)])
def test_prefill_call_in_a_graph(m, n, k):
    wq, ws, _ = pdq.quantize_weight(dev(synth.weights(8200, n, k, "bf16"), "bf16"))
    bias = torch.from_numpy(synth.bias(8201, n)).cuda()
    x_static = torch.empty((m, k), dtype=torch.bfloat16, device="cuda")
    inputs = [_x(8210 + i, m, k, cols=(3 + i, k - 1)) for i in range(REPLAYS)]

    def call(x):
        return pdq.linear_prefill(x, wq, ws, bias, want_acc=True)

    def compare(got, ref, i):
        _same(got["y"], ref["y"], f"y, replay {i}")
        _same(got["acc"], ref["acc"], f"acc, replay {i}")
        _same(got["x_scale"], ref["x_scale"], f"scales, replay {i}")
        assert torch.equal(got["xq"].data, ref["xq"].data), f"codes, replay {i}"

    _replay_against_eager(call, x_static, inputs, compare)


def test_int8_outlier_noalloc_in_a_graph():
    """A different outlier set on every replay (2, 5 and 0 columns), so that the
    count, the column list and the gathered operands change between replays."""
    m, n, k = 256, 512, 1024
    w16 = dev(synth.weights(8300, n, k, "f16"), "f16")
    wq, ws, _ = pdq.quantize_weight(w16)
    bias = torch.from_numpy(synth.bias(8301, n)).cuda()
    x_static = torch.empty((m, k), dtype=torch.float16, device="cuda")
    sets = [(11, 600), (0, 64, 65, 512, 1023), ()]
    inputs = [_x(8310 + i, m, k, "f16", cols, 60.0) for i, cols in enumerate(sets)]

    def call(x):
        return pdq.linear_int8_outlier_noalloc(x, 6.0, wq, ws, w16, bias, max_outliers=64, want_acc=True)

    def compare(got, ref, i):
        cnt = int(host(got["count"])[0])
        assert cnt == int(host(ref["count"])[0]) == len(sets[i]), f"count, replay {i}"
        assert host(got["idx"])[:cnt].tolist() == sorted(sets[i]), f"columns, replay {i}"
        _same(got["y"], ref["y"], f"y, replay {i}")
        _same(got["acc"], ref["acc"], f"acc, replay {i}")
        _same(got["x_scale"], ref["x_scale"], f"scales, replay {i}")
        assert torch.equal(got["xq"].data, ref["xq"].data), f"codes, replay {i}"

    _replay_against_eager(call, x_static, inputs, compare)
