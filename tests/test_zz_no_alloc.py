"""pdq_linear_int8_outlier_noalloc (the LLM.int8 call on the library's own
scratch, for callers that cannot allocate) against pdq_linear_int8_outlier
with a caller workspace, through the C ABI: every output bit for bit, on
consecutive calls whose second is smaller than the first (the scratch then
still holds the first call's bytes), and against the oracle's outlier set."""
import numpy as np
import pytest
import torch

import oracle.pdq_oracle as O
from w8a8_int8_quantized_absmax_amd import pdq, synth
from gpu_helpers import dev, host

pytestmark = pytest.mark.gpu


def _case(seed, m, n, k, cols, dtype):
    x = synth.normal(seed, (m, k))
    x[:, cols] = synth.normal(seed + 1, (m, len(cols)), 60.0)
    x = synth.round_to(x, dtype)
    w = synth.weights(seed + 2, n, k, dtype)
    return x, w


def _compare(x, w, dtype, max_out=64):
    xd, wd = dev(x, dtype), dev(w, dtype)
    wq, ws, _ = pdq.quantize_weight(wd)
    bias = torch.from_numpy(synth.bias(77, w.shape[0])).cuda()
    ref = pdq.linear_int8_outlier(xd, 6.0, wq, ws, wd, bias, max_outliers=max_out, want_acc=True)
    got = pdq.linear_int8_outlier_noalloc(xd, 6.0, wq, ws, wd, bias, max_outliers=max_out, want_acc=True)
    torch.cuda.synchronize()
    cnt = int(host(got["count"])[0])
    assert cnt == int(host(ref["count"])[0])
    cols = O.outlier_columns(x, 6.0)
    assert cnt == len(cols) and host(got["idx"])[:cnt].tolist() == cols.tolist()
    assert np.array_equal(host(got["idx"])[:cnt], host(ref["idx"])[:cnt])
    assert torch.equal(got["xq"].data[:pdq.act_bytes(*x.shape)], ref["xq"].data[:pdq.act_bytes(*x.shape)])
    assert torch.equal(got["x_scale"].view(torch.int32), ref["x_scale"].view(torch.int32))
    assert torch.equal(got["acc"], ref["acc"])
    assert torch.equal(got["y"].view(torch.int16), ref["y"].view(torch.int16))
    return cnt


def test_noalloc_matches_workspace_call_twice_second_smaller():
    k1 = 4096
    x1, w1 = _case(9700, 512, 8192, k1, [5, 700, 4000, 4095], "f16")
    x2, w2 = _case(9710, 37, 300, 1040, [0, 333, 1039], "f16")
    assert _compare(x1, w1, "f16") == 4
    assert _compare(x2, w2, "f16") == 3
    # and once more the first problem, in bf16, after the smaller one
    x3, w3 = _case(9720, 512, 8192, k1, [1, 2048], "bf16")
    assert _compare(x3, w3, "bf16") == 2


def test_noalloc_refuses_a_problem_beyond_its_scratch():
    x = torch.zeros((4, 64), dtype=torch.float16, device="cuda")
    n = 70000
    need = pdq.int8_outlier_workspace_bytes(2048, n, 8192, 64)
    assert need > pdq.noalloc_scratch_bytes()
    with pytest.raises(pdq.PdqError) as e:
        pdq._call("pdq_linear_int8_outlier_noalloc", pdq._p(x), pdq.F16, 2048, 8192, 8192, 6.0, pdq._p(x),
                  pdq._p(x), pdq._p(x), 8192, None, n, pdq._p(x), n, pdq._p(x), pdq._p(x), pdq._p(x),
                  pdq._p(x), 64, None, pdq._stream(x.device))
    assert e.value.status == 6  # PDQ_ERR_WORKSPACE, before anything is enqueued
