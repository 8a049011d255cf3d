"""fa_bwd_noalloc (the backward entry point that allocates nothing and uses
the library's static device scratch) against fa_bwd_gqa with a caller
workspace, through the C ABI: two calls in a row on one device, the second
smaller, so the second runs on scratch the first left behind. bf16 gradients
are bitwise deterministic, so they must be identical; fp32 dQ is summed with
atomics, so it is compared at the fp32 bound."""

import numpy as np
import pytest
import torch

from exact_io_aware_fa_amd import binding as B
from exact_io_aware_fa_amd.inputs import custom, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def _run(w, noalloc):
    inp = make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v, do = (inp[x].to(dev) for x in ("q", "k", "v", "do"))
    kvl = None if inp["kv_len"] is None else inp["kv_len"].to(dev)
    b, h, n, d = q.shape
    hkv = k.shape[1]
    dt = B.FA_BF16 if q.dtype == torch.bfloat16 else B.FA_FP32
    stream = torch.cuda.current_stream().cuda_stream
    o = torch.empty_like(q)
    lse = torch.empty((b, h, n), dtype=torch.float32, device=dev)
    kp = None if kvl is None else kvl.data_ptr()
    B.check(B.fa_fwd_gqa(b, h, hkv, n, d, w.causal, w.softmax_scale, dt, q.data_ptr(),
                         k.data_ptr(), v.data_ptr(), kp, o.data_ptr(), lse.data_ptr(), stream))
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    args = (b, h, hkv, n, d, w.causal, w.softmax_scale, dt, q.data_ptr(), k.data_ptr(),
            v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(), kp, dq.data_ptr(),
            dk.data_ptr(), dv.data_ptr())
    if noalloc:
        B.check(B.fa_bwd_noalloc(*args, stream))
    else:
        wsb = B.fa_bwd_workspace_bytes(b, h, n, d, dt)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        B.check(B.fa_bwd_gqa(*args, ws.data_ptr(), wsb, stream))
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


CASES = [
    # (name, batch, heads, heads_kv, n, d, dtype, causal, padded)
    [("big", 2, 8, 4, 1000, 128, "bf16", True, False), ("small", 1, 2, 2, 129, 64, "bf16", False,
                                                         True)],
    [("big", 1, 4, 4, 700, 256, "bf16", False, True), ("small", 2, 2, 1, 65, 128, "bf16", True,
                                                       False)],
    [("big", 1, 2, 2, 300, 64, "fp32", True, True), ("small", 1, 1, 1, 50, 64, "fp32", False,
                                                     False)],
    # From 4096 rows, d = 128 runs the 64-keys-per-wave dK/dV kernel.
    [("big", 1, 4, 2, 4200, 128, "bf16", True, True), ("small", 1, 2, 2, 4100, 128, "bf16",
                                                        False, False)],
]


@pytest.mark.parametrize("pair", CASES)
def test_noalloc_matches_workspace_call_twice(pair):
    for name, b, h, hkv, n, d, dt, causal, padded in pair:
        w = custom(f"noalloc_{name}_n{n}_d{d}", b, h, n, d, dt, causal, seed=n + d,
                   padded=padded, heads_kv=hkv)
        print(f"[noalloc] {name} b={b} h={h} hkv={hkv} n={n} d={d} {dt} causal={causal} "
              f"padded={padded}", flush=True)
        got = _run(w, True)
        ref = _run(w, False)
        for g, r, nm in zip(got, ref, ("dq", "dk", "dv")):
            if dt == "bf16":
                assert torch.equal(g, r), nm
            else:
                gg, rr = g.double().numpy(), r.double().numpy()
                err = np.abs(gg - rr).max() / max(np.abs(rr).max(), 1e-30)
                assert err <= 1e-5, (nm, err)


def test_noalloc_rejects_calls_beyond_the_scratch():
    # 80 heads x 32768 rows: two fp32 vectors of 10 MiB each exceed 16 MiB.
    need = B.fa_bwd_workspace_bytes(1, 80, 32768, 128, B.FA_BF16)
    assert need > B.FA_NOALLOC_SCRATCH_BYTES
    stream = torch.cuda.current_stream().cuda_stream
    fake = [0x1000_0000 * (i + 1) for i in range(9)]
    st = B.fa_bwd_noalloc(1, 80, 80, 32768, 128, 1, 0.088, B.FA_BF16, *fake[:6], None,
                          *fake[6:9], stream)
    assert st == B.FA_E_SCRATCH
