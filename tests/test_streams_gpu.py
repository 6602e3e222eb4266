"""Every entry point enqueues on the stream it is given.

Each call runs once on the default stream (the reference) and once on a
side stream right after that stream has filled the call's outputs with NaN
(or 0xff codes).  A call that ignored its stream argument could race the
fill; in stream order the outputs must equal the reference bit for bit (the
kernels are deterministic).  Streams keep the default priority.
"""
import sys

import pytest
import torch

from io_aware_exact_05_amd import inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _fa():
    from io_aware_exact_05_amd import fa
    return fa


def _on_side_stream(fill, call, outs):
    """fill() and call(stream) in order on a new stream; returns clones of outs."""
    main = torch.cuda.current_stream()
    s = torch.cuda.Stream()
    s.wait_stream(main)
    with torch.cuda.stream(s):
        fill()
        call(s)
    main.wait_stream(s)
    torch.cuda.synchronize()
    return [t.clone() for t in outs]


def _same(a, b):
    return all(torch.equal(x.view(torch.uint8), y.view(torch.uint8)) for x, y in zip(a, b))


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("causal", [0, 1])
def test_forward_on_a_side_stream(dtype, causal):
    _say(f"case stream forward dtype={dtype} causal={causal}")
    fa = _fa()
    q, k, v = (t.cuda() for t in inputs.random_inputs(2, 8, 1000, 128, dtype, seed=31))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device="cuda")
    fa.fa_fwd(q, k, v, o, lse, bool(causal), 0.088)
    torch.cuda.synchronize()
    ref = [o.clone(), lse.clone()]

    def fill():
        o.fill_(float("nan"))
        lse.fill_(float("nan"))

    got = _on_side_stream(fill, lambda s: fa.fa_fwd(q, k, v, o, lse, bool(causal), 0.088, s),
                          [o, lse])
    assert _same(got, ref)


@pytest.mark.parametrize("causal", [0, 1])
def test_backward_on_a_side_stream(causal):
    _say(f"case stream backward causal={causal}")
    fa = _fa()
    q, k, v = (t.cuda() for t in inputs.random_inputs(2, 8, 700, 128, "bf16", seed=37))
    dout = inputs.random_inputs(2, 8, 700, 128, "bf16", seed=38)[0].cuda()
    o, lse = fa.attention(q, k, v, bool(causal), 0.088)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.bwd_workspace_bytes(2, 8, 700), dtype=torch.uint8, device="cuda")
    fa.fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, ws, bool(causal), 0.088)
    torch.cuda.synchronize()
    ref = [dq.clone(), dk.clone(), dv.clone()]

    def fill():
        for t in (dq, dk, dv):
            t.fill_(float("nan"))
        ws.fill_(255)

    got = _on_side_stream(
        fill, lambda s: fa.fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, ws, bool(causal), 0.088, s),
        [dq, dk, dv])
    assert _same(got, ref)


@pytest.mark.parametrize("causal", [0, 1])
def test_fp8_quantiser_and_attention_on_a_side_stream(causal):
    _say(f"case stream fp8 causal={causal}")
    fa = _fa()
    B, H, N, d = 1, 8, 1000, 128
    q, k, v = (t.cuda() for t in inputs.random_inputs(B, H, N, d, "f32", seed=41))
    signs = inputs.rotation_signs(d, seed=0).cuda()
    nb = -(-N // 128)
    codes = [torch.empty((B, H, N, d), dtype=torch.uint8, device="cuda") for _ in range(3)]
    descs = [torch.empty((B, H, nb), dtype=torch.float32, device="cuda") for _ in range(3)]
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")

    def call(s):
        for x, c, ds, rot in zip((q, k, v), codes, descs, (True, True, False)):
            fa.fa_quantize_e4m3(x, c, ds, rot, signs if rot else None, s)
        fa.fa_fwd_fp8(*codes, *descs, o, lse, bool(causal), 0.088, s)

    call(None)
    torch.cuda.synchronize()
    outs = codes + descs + [o, lse]
    ref = [t.clone() for t in outs]

    def fill():
        for c in codes:
            c.fill_(255)
        for t in descs + [o, lse]:
            t.fill_(float("nan"))

    got = _on_side_stream(fill, call, outs)
    assert _same(got, ref)


@pytest.mark.parametrize("causal", [0, 1])
def test_decoding_on_a_side_stream(causal):
    _say(f"case stream decoding causal={causal}")
    fa = _fa()
    B, H, Hkv, Nq, Nkv, d = 2, 8, 2, 4, 5000, 128
    q = inputs.random_inputs(B, H, Nq, d, "bf16", seed=43)[0].cuda()
    _, k, v = (t.cuda() for t in inputs.random_inputs(B, Hkv, Nkv, d, "bf16", seed=44))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device="cuda")
    wb = fa.kvcache_workspace_bytes(B, H, Hkv, Nq, Nkv, d)
    ws = torch.empty(max(wb, 1), dtype=torch.uint8, device="cuda") if wb else None
    fa.fa_fwd_kvcache(q, k, v, o, lse, ws, bool(causal), 0.088)
    torch.cuda.synchronize()
    ref = [o.clone(), lse.clone()]

    def fill():
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        if ws is not None:
            ws.fill_(255)

    got = _on_side_stream(
        fill, lambda s: fa.fa_fwd_kvcache(q, k, v, o, lse, ws, bool(causal), 0.088, s), [o, lse])
    assert _same(got, ref)
