"""GPU parity for packed variable-length batches (page 2, "4. FlashAttention
深度剖析", 4.7.2 and 4.7.4: variable-length sequences without padding).

Sequences are stored back to back per head ([heads, total, d]); each attends
only to itself, causal positions counted from its first row. Small batches
(an empty and a one-row sequence among them, grouped heads, d = 64/128/256,
bf16 and fp32, and two d = 128 batches whose longest sequence passes 4096
rows) are compared with the fp64 oracle per (head, sequence). At
the measured size (32 heads, 16384 packed rows, lengths 256..4096, d = 128,
causal) every output is compared bit for bit with the padded-layout call on
each sequence on its own (the same kernels on the same rows), and seeded
rows against the oracle. Rows outside every sequence are left unwritten.
"""

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_fa_amd import attention as fa
from exact_io_aware_fa_amd import binding as B
from exact_io_aware_fa_amd.inputs import PACKED, PackedWorkload, make_packed_inputs
from parity_utils import BF16_GRAD_REL, BF16_LSE_ABS, BF16_O_ABS, FP32_REL, f64, normwise_rel

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def _packed(name, heads, heads_kv, lengths, d, causal, dtype, seed):
    return PackedWorkload(name, heads, heads_kv, sum(lengths), (1, 1), d, dtype, causal, seed,
                          lengths=tuple(lengths))


def _run(w, inp):
    q, k, v, do = (inp[x].cuda() for x in ("q", "k", "v", "do"))
    cu = inp["cu_seqlens"]
    o, lse = fa.flash_attn_varlen_fwd(q, k, v, cu, None, w.causal, w.softmax_scale)
    dq, dk, dv = fa.flash_attn_varlen_bwd(q, k, v, o, lse, do, cu, None, w.causal,
                                          w.softmax_scale)
    torch.cuda.synchronize()
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


SMALL = [
    # (heads, heads_kv, lengths, d, causal, dtype)
    (4, 4, (5, 1, 0, 130, 64, 300), 64, True, "bf16"),
    (4, 2, (129, 5, 700), 64, False, "bf16"),
    (2, 1, (1500, 40), 64, True, "bf16"),
    (4, 2, (257, 3, 100), 128, False, "bf16"),
    (4, 1, (129, 383, 7), 256, True, "bf16"),
    (2, 2, (1000, 24), 128, True, "bf16"),
    # Longest sequence from 4096 rows: the 64-keys-per-wave dK/dV kernel,
    # whose 256-key workgroups past a shorter sequence's end exit at once.
    (2, 1, (4500, 300, 0, 37), 128, True, "bf16"),
    (2, 2, (129, 4200), 128, False, "bf16"),
    (4, 4, (300, 1, 65), 128, True, "fp32"),
    (2, 2, (31, 200), 256, False, "fp32"),
    (6, 3, (64, 64, 0, 64, 500), 64, False, "fp32"),
]


@pytest.mark.parametrize("heads,heads_kv,lengths,d,causal,dtype", SMALL)
def test_packed_against_oracle(heads, heads_kv, lengths, d, causal, dtype):
    w = _packed("varlen_small", heads, heads_kv, lengths, d, causal, dtype,
                seed=sum(lengths) + d + heads)
    inp = make_packed_inputs(w)
    print(f"[parity] varlen heads={heads} kv={heads_kv} lengths={lengths} d={d} "
          f"causal={causal} {dtype}", flush=True)
    gpu = _run(w, inp)
    cu = [int(x) for x in inp["cu_seqlens"]]
    args = [f64(inp[x]) for x in ("q", "k", "v")]
    o, lse = oracle.varlen_fwd(*args, cu, causal, w.softmax_scale)
    dq, dk, dv = oracle.varlen_bwd(*args, f64(inp["do"]), cu, causal, w.softmax_scale)
    go, gl = f64(gpu["o"]), gpu["lse"].cpu().double().numpy()
    grads = {"dq": (f64(gpu["dq"]), dq), "dk": (f64(gpu["dk"]), dk), "dv": (f64(gpu["dv"]), dv)}
    tol = FP32_REL if dtype == "fp32" else BF16_GRAD_REL
    for a, e in zip(cu[:-1], cu[1:]):
        if e == a:
            continue
        for h in range(heads):
            if dtype == "fp32":
                assert normwise_rel(go[h, a:e], o[h, a:e]) <= FP32_REL, (h, a)
                assert np.all(np.abs(gl[h, a:e] - lse[h, a:e])
                              <= FP32_REL * np.maximum(1.0, np.abs(lse[h, a:e])))
            else:
                assert np.abs(go[h, a:e] - o[h, a:e]).max() <= BF16_O_ABS, (h, a)
                assert np.abs(gl[h, a:e] - lse[h, a:e]).max() <= BF16_LSE_ABS, (h, a)
            assert normwise_rel(grads["dq"][0][h, a:e], grads["dq"][1][h, a:e]) <= tol, (h, a)
        for j in range(heads_kv):
            for name in ("dk", "dv"):
                got, ref = grads[name]
                assert normwise_rel(got[j, a:e], ref[j, a:e]) <= tol, (name, j, a)


def test_packed_equals_per_sequence_calls_at_full_size():
    w = PACKED["varlen_causal_h32_t16384_d128"]
    inp = make_packed_inputs(w)
    print(f"[parity] {w.name}: packed vs per-sequence calls", flush=True)
    gpu = _run(w, inp)
    cu = [int(x) for x in inp["cu_seqlens"]]
    q, k, v, do = (inp[x].cuda() for x in ("q", "k", "v", "do"))
    for a, e in zip(cu[:-1], cu[1:]):
        sl = [x[:, a:e].unsqueeze(0).contiguous() for x in (q, k, v, do)]
        o, lse = fa.flash_attn_fwd(sl[0], sl[1], sl[2], True, w.softmax_scale)
        dq, dk, dv = fa.flash_attn_bwd(sl[0], sl[1], sl[2], o, lse, sl[3], True, w.softmax_scale)
        torch.cuda.synchronize()
        for name, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
            assert torch.equal(gpu[name][:, a:e], t[0]), (name, a, e)
    # Seeded rows of a few (head, sequence) pairs against the oracle.
    rng = np.random.default_rng(w.seed)
    for h, s in ((0, 0), (17, len(cu) // 2), (31, len(cu) - 2)):
        a, e = cu[s], cu[s + 1]
        rows = np.sort(rng.choice(e - a, size=min(16, e - a), replace=False))
        ref = oracle.head_forward(f64(inp["q"][h, a:e]), f64(inp["k"][h, a:e]),
                                  f64(inp["v"][h, a:e]), w.softmax_scale, True, rows=rows)
        go = f64(gpu["o"][h, a:e])[rows]
        gl = gpu["lse"][h, a:e].cpu().double().numpy()[rows]
        assert np.abs(go - ref["o"]).max() <= BF16_O_ABS
        assert np.abs(gl - ref["lse"]).max() <= BF16_LSE_ABS


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_rows_outside_every_sequence_are_not_written(dtype):
    # Offsets that stop 37 rows short of the total: those rows of every
    # output keep what the caller put there.
    heads, total, d, tail = 2, 300, 64, 37
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dt = B.FA_BF16 if dtype == "bf16" else B.FA_FP32
    g = torch.Generator().manual_seed(3)
    q, k, v, do = (torch.randn(heads, total, d, generator=g).to(tdt).cuda() for _ in range(4))
    cu = torch.tensor([0, 100, total - tail], dtype=torch.int32).cuda()
    o = torch.full_like(q, 7.0)
    lse = torch.full((heads, total), 7.0, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    B.check(B.fa_fwd_varlen(2, heads, heads, total, 163, d, cu.data_ptr(), 1, 0.125, dt,
                            q.data_ptr(), k.data_ptr(), v.data_ptr(), None, o.data_ptr(),
                            lse.data_ptr(), s))
    grads = [torch.full_like(q, 7.0) for _ in range(3)]
    wsb = B.fa_bwd_workspace_bytes(2, heads, 163, d, dt)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    B.check(B.fa_bwd_varlen(2, heads, heads, total, 163, d, cu.data_ptr(), 1, 0.125, dt,
                            q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                            do.data_ptr(), lse.data_ptr(), None, *(t.data_ptr() for t in grads),
                            ws.data_ptr(), wsb, s))
    torch.cuda.synchronize()
    for t in [o, lse] + grads:
        assert torch.all(t[:, total - tail:] == 7.0)
        assert torch.isfinite(t[:, :total - tail]).all()
        assert not torch.all(t[:, :total - tail] == 7.0)


def test_autograd_wrapper_and_argument_checks():
    w = _packed("varlen_autograd", 2, 1, (50, 77), 64, True, "bf16", seed=8)
    inp = make_packed_inputs(w)
    q, k, v, do = (inp[x].cuda() for x in ("q", "k", "v", "do"))
    cu = inp["cu_seqlens"]
    qr, kr, vr = (x.clone().requires_grad_(True) for x in (q, k, v))
    o = fa.flash_attention_varlen(qr, kr, vr, cu, causal=True)
    o.backward(do)
    o2, lse = fa.flash_attn_varlen_fwd(q, k, v, cu, causal=True)
    dq, dk, dv = fa.flash_attn_varlen_bwd(q, k, v, o2, lse, do, cu, causal=True)
    assert torch.equal(o, o2) and torch.equal(qr.grad, dq)
    assert torch.equal(kr.grad, dk) and torch.equal(vr.grad, dv)
    with pytest.raises(ValueError):
        fa.flash_attn_varlen_fwd(q, k, v, [0, 50, 126])      # does not end at total
    with pytest.raises(ValueError):
        fa.flash_attn_varlen_fwd(q, k, v, [0, 80, 50, 127])  # decreasing
    with pytest.raises(ValueError):
        fa.flash_attn_varlen_fwd(q, k, v, cu, max_seqlen=60)  # below the longest
