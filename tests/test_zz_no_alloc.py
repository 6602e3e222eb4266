"""GPU test of fa_fwd_kvcache_noalloc, the key/value-cache pass whose
workspace is the library's static per-device scratch, for callers that
cannot allocate.  Through the C ABI it must give exactly what
fa_fwd_kvcache gives with a caller workspace (same kernels, same cut of the
cache): O and LSE bit for bit, and both within the forward gates of the fp64
KV-cache oracle.  Three calls in a row: the first fills the scratch, the
second (smaller, another dtype and head dimension) must not see stale
partial results from it, the third takes the largest workspace any valid
shape needs.  The calls allocate no device memory."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from gates import check, widen
from io_aware_exact_05_amd import inputs

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "f16": torch.float16}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _inputs(B, H, Hkv, Nq, Nkv, d, dtype, seed):
    q, _, _ = inputs.random_inputs(B, H, Nq, d, dtype, seed)
    _, k, v = inputs.random_inputs(B, Hkv, Nkv, d, dtype, seed + 1)
    return q, k, v


def _run_both(q, k, v, causal, scale):
    """(o, lse) of fa_fwd_kvcache with a torch workspace, then of the
    no-allocation entry point, both through the C ABI on the current stream."""
    from io_aware_exact_05_amd import fa
    B, H, Nq, d = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    need = fa.kvcache_workspace_bytes(B, H, Hkv, Nq, Nkv, d)
    assert 0 < need <= fa.KVCACHE_SCRATCH_BYTES
    code = fa.DTYPE_CODE[q.dtype]
    stream = torch.cuda.current_stream().cuda_stream
    o1, o2 = torch.full_like(q, float("nan")), torch.full_like(q, float("nan"))
    l1 = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device=q.device)
    l2 = torch.full_like(l1, float("nan"))
    ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = fa.fa_fwd_kvcache_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o1.data_ptr(), l1.data_ptr(),
                               ws.data_ptr(), need, B, H, Hkv, Nq, Nkv, d, causal, scale, code, stream)
    assert st == 0, fa.status_string(st)
    torch.cuda.synchronize()
    before = (torch.cuda.mem_get_info()[0], torch.cuda.memory_allocated())
    st = fa.fa_fwd_kvcache_noalloc_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o2.data_ptr(),
                                       l2.data_ptr(), B, H, Hkv, Nq, Nkv, d, causal, scale, code, stream)
    assert st == 0, fa.status_string(st)
    torch.cuda.synchronize()
    after = (torch.cuda.mem_get_info()[0], torch.cuda.memory_allocated())
    return o1, l1, o2, l2, before, after


CALLS = [  # B, H, Hkv, Nq, Nkv, d, dtype, causal, seed
    (2, 16, 4, 4, 8229, 128, "bf16", 1, 101),   # 4 x 4 rows per K/V head, several chunks, ragged
    (1, 8, 8, 1, 3000, 64, "f16", 0, 202),      # smaller workspace, other dtype and d
    (255, 32, 1, 1, 1024, 256, "bf16", 1, 303),  # the largest workspace of any cut (16320 partial rows)
]


def test_noalloc_matches_workspace_entry_point_on_consecutive_calls():
    from io_aware_exact_05_amd import fa
    prev_need = None
    for i, (B, H, Hkv, Nq, Nkv, d, dtype, causal, seed) in enumerate(CALLS):
        what = f"noalloc call {i}: {dtype} B={B} H={H} Hkv={Hkv} Nq={Nq} Nkv={Nkv} d={d} causal={causal}"
        _say(f"case {what}")
        need = fa.kvcache_workspace_bytes(B, H, Hkv, Nq, Nkv, d)
        if i == 1:
            assert need < prev_need, "the second call must use a smaller workspace"
        prev_need = need
        q, k, v = _inputs(B, H, Hkv, Nq, Nkv, d, dtype, seed)
        scale = float(np.float32(1 / math.sqrt(d)))
        o1, l1, o2, l2, before, after = _run_both(q.cuda(), k.cuda(), v.cuda(), causal, scale)
        if i > 0:  # code objects and the scratch address are loaded by now
            assert after == before, f"{what}: device memory changed {before} -> {after}"
        assert torch.equal(o1, o2), f"{what}: O differs from fa_fwd_kvcache"
        assert torch.equal(l1, l2), f"{what}: LSE differs from fa_fwd_kvcache"
        if B * H * Nq <= 4096:  # whole oracle
            o_ref, l_ref = oracle.attention_kvcache(widen(q), widen(k), widen(v), causal, scale)
            st = check(o2.cpu(), l2.cpu(), o_ref, l_ref, dtype, what)
        else:  # every row of a few batch entries
            sel = [0, B // 2, B - 1]
            o_ref, l_ref = oracle.attention_kvcache(widen(q[sel]), widen(k[sel]), widen(v[sel]), causal,
                                                    scale)
            st = check(o2[sel].cpu(), l2[sel].cpu(), o_ref, l_ref, dtype, what + f" batches {sel}")
        _say(f"  {st}")


def test_noalloc_single_chunk_needs_no_scratch():
    from io_aware_exact_05_amd import fa
    _say("case noalloc single chunk")
    q, k, v = (x.cuda() for x in _inputs(2, 4, 2, 1, 300, 128, "bf16", 404))
    assert fa.kvcache_workspace_bytes(2, 4, 2, 1, 300, 128) == 0
    o1, l1 = fa.attention_kvcache(q, k, v, True, 0.088)
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    fa.fa_fwd_kvcache_noalloc(q, k, v, o2, l2, True, 0.088)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
