"""The library's calls running concurrently on separate streams.

The library holds no mutable global state, and every call enqueues its
kernels on the stream it is given: calls on different streams may overlap
on the GPU, and each must still give exactly the outputs it gives alone.
Four different calls (per-token prefill on the tiled GEMM, static decode on
the skinny kernel, per-token asymmetric prefill, LLM.int8 with its own
workspace) are each run once on the default stream, then three times each
on four streams at once, interleaved; every output must equal the lone
call's bit for bit.  (Parity of the lone calls with the oracle is
established by the other GPU tests.)"""
import numpy as np
import pytest
import torch

import oracle.pdq_oracle as O
from w8a8_int8_quantized_absmax_amd import pdq, synth
from gpu_helpers import dev

pytestmark = pytest.mark.gpu

REPEATS = 3


def _bits(t):
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16)
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    return t


def _outputs(res):
    """The tensors of a call's result dict (packed codes by their bytes)."""
    out = {}
    for k, v in res.items():
        if isinstance(v, pdq.Codes):
            out[k] = v.data
        elif isinstance(v, torch.Tensor):
            out[k] = v
    return out


def test_concurrent_calls_on_four_streams_equal_lone_calls():
    # prefill, per-token symmetric: 2048 x 2600 x 1040 runs on the tiled GEMM
    xp = dev(synth.activations(9700, 2048, 1040, [3, 500], 100.0), "bf16")
    wp = pdq.quantize_weight(dev(synth.weights(9701, 2600, 1040), "bf16"))
    # decode, static asymmetric at 32 rows: the skinny kernel
    cal = [synth.activations(9710 + b, 64, 4096, [1, 4000], 100.0, offset=0.1) for b in range(3)]
    _, s, z = O.calibrate(cal)
    xd = dev(synth.activations(9720, 32, 4096, [1, 4000], 100.0, offset=0.1), "bf16")
    wd = pdq.quantize_weight(dev(synth.weights(9721, 4096, 4096), "bf16"))
    # per-token asymmetric prefill
    xa = dev(synth.activations(9730, 600, 2048, [7], 100.0, offset=0.3), "bf16")
    wa = pdq.quantize_weight(dev(synth.weights(9731, 1500, 2048), "bf16"))
    # LLM.int8 (each call with its own workspace, allocated by the binding)
    xo_h = synth.normal(9740, (512, 2048))
    cols = synth.choose_channels(9741, 2048, 8)
    xo_h[:, cols] = synth.normal(9742, (512, 8), 60.0)
    xo = dev(synth.round_to(xo_h, "f16"), "f16")
    wo16 = dev(synth.weights(9743, 3000, 2048, "f16"), "f16")
    wo = pdq.quantize_weight(wo16)

    calls = [
        lambda: pdq.linear_prefill(xp, wp[0], wp[1], want_acc=True),
        lambda: pdq.linear_decode(xd, s, z, wd[0], wd[1], wd[2], want_acc=True),
        lambda: pdq.linear_prefill_asym(xa, wa[0], wa[1], wa[2], want_acc=True),
        lambda: pdq.linear_int8_outlier(xo, 6.0, wo[0], wo[1], wo16, want_acc=True),
    ]
    torch.cuda.synchronize()
    ref = [_outputs(c()) for c in calls]
    torch.cuda.synchronize()

    streams = [torch.cuda.Stream() for _ in calls]
    main = torch.cuda.current_stream()
    for st in streams:
        st.wait_stream(main)
    got = [[] for _ in calls]
    for _ in range(REPEATS):
        for i, (st, c) in enumerate(zip(streams, calls)):
            with torch.cuda.stream(st):
                got[i].append(_outputs(c()))
    torch.cuda.synchronize()
    for i, runs in enumerate(got):
        for r, out in enumerate(runs):
            assert out.keys() == ref[i].keys()
            for k in out:
                a, b = out[k], ref[i][k]
                if k == "idx":  # entries past the count are unset
                    cnt = int(ref[i]["count"].item())
                    a, b = a[:cnt], b[:cnt]
                assert torch.equal(_bits(a), _bits(b)), f"call {i} repeat {r}: {k} differs"
    assert int(ref[3]["count"].item()) == len(cols)
    assert np.array_equal(ref[3]["idx"][:len(cols)].cpu().numpy(), cols)
