"""attn_bwd_noalloc (the allocation-free backward: row statistics in the
library's own per-GPU array) against attn_bwd (caller workspace) and the fp64
oracle, through the C ABI (needs the GPU).

Three calls in a row on one GPU, each smaller than the one before: the first
fills the array to its limit (2^20 rows), the later ones reuse it with fewer
rows, so stale contents of an earlier call must not leak into a later one.
Every gradient must equal attn_bwd's bit for bit (same kernels, same inputs);
the two smaller calls are also held to the oracle's gradient bars.
"""
import numpy as np
import pytest

from oracle import attention_bwd, bf16_bits_to_f64, check_grads
from workloads import make_dout, make_random

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tiled_attention_16_amd as ta
    ta.load_library()
    return ta


def to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def f64(t):
    return bf16_bits_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))


CALLS = [
    # B, H, N_q, N_k, d, causal, seqlens_k, q_start, oracle
    (1, 256, 4096, 64, 64, 0, None, None, False),          # B*H*N_q = 2^20 rows, the limit
    (2, 3, 700, 650, 128, 1, [650, 333], [0, 70], True),
    (1, 2, 300, 300, 64, 2, None, None, True),
]


def test_noalloc_matches_attn_bwd_on_successive_calls():
    import tiled_attention_16_amd as ta
    for i, (B, H, nq, nk, d, causal, sl, qs, use_oracle) in enumerate(CALLS):
        print(f"  call {i}: B,H,Nq,Nk,d={B},{H},{nq},{nk},{d} causal={causal} rows={B * H * nq}", flush=True)
        q, k, v = make_random(B, H, nq, nk, d, seed=400 + i)
        g = make_dout((B, H, nq, d), seed=500 + i)
        scale = float(np.float32(d ** -0.5))
        tsl = torch.tensor(sl, dtype=torch.int32, device="cuda") if sl is not None else None
        tqs = torch.tensor(qs, dtype=torch.int32, device="cuda") if qs is not None else None
        tq, tk, tv, tg = to_dev(q), to_dev(k), to_dev(v), to_dev(g)
        o, lse = ta.attn_fwd(tq, tk, tv, causal=causal, scale=scale, seqlens_k=tsl, q_start=tqs)
        rq, rk, rv = ta.attn_bwd(tq, tk, tv, o, lse, tg, causal=causal, scale=scale, seqlens_k=tsl, q_start=tqs)
        nq_, nk_, nv_ = (torch.full_like(t, float("nan")) for t in (tq, tk, tv))
        dq, dk, dv = ta.attn_bwd_noalloc(tq, tk, tv, o, lse, tg, nq_, nk_, nv_, causal=causal, scale=scale,
                                         seqlens_k=tsl, q_start=tqs)
        torch.cuda.synchronize()
        for name, a, b in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"call {i}: {name} differs from attn_bwd"
        if use_oracle:
            eq, ek, ev = attention_bwd(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v),
                                       bf16_bits_to_f64(g), scale, causal,
                                       seqlens_k=None if sl is None else np.array(sl),
                                       q_start=None if qs is None else np.array(qs))
            r = check_grads({"dq": f64(dq), "dk": f64(dk), "dv": f64(dv)}, {"dq": eq, "dk": ek, "dv": ev})
            print(f"  call {i}: {r}", flush=True)
            assert r.ok, f"call {i}: {r}"


def test_noalloc_rejects_rows_beyond_the_limit():
    import tiled_attention_16_amd as ta
    # one row past 2^20: refused on the host before anything runs
    t = torch.empty((1, 16, 65537, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((1, 16, 8, 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, 16, 65537), dtype=torch.float32, device="cuda")
    with pytest.raises(ta.AttnError) as e:
        ta.attn_bwd_noalloc(t, k, k.clone(), t.clone(), lse, t.clone(), t.clone(), k.clone(), k.clone())
    assert e.value.status == ta.ATTN_ERR_SCRATCH
