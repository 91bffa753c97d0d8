"""Parity of the HIP attention backward (attn_bwd) with the fp64 CPU oracle (needs the GPU).

The forward (attn_fwd) runs on the GPU to give O and LSE, as in training; the
oracle computes dQ, dK, dV from the bf16 inputs alone (it takes neither O nor
LSE from the GPU). Bars (oracle/checker.py): per gradient, max |d| <= 2e-2 *
max(1, max |ref|) and mean |d| <= 1e-2 * mean |ref| + 1e-6.
"""
import numpy as np
import pytest

from oracle import attention_bwd, bf16_bits_to_f64, check_grads
from workloads import WORKLOADS, make_dout, make_inputs, make_random

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


def run_bwd(q, k, v, g, scale, causal, seqlens=None, qstart=None):
    import tiled_attention_16_amd as ta
    print(f"  bwd B,H,Nq,Nk,d={q.shape[0]},{q.shape[1]},{q.shape[2]},{k.shape[2]},{q.shape[3]} causal={causal} "
          f"seqlens={seqlens is not None} q_start={qstart is not None}", flush=True)
    sl = torch.from_numpy(np.asarray(seqlens, np.int32)).cuda() if seqlens is not None else None
    qs = torch.from_numpy(np.asarray(qstart, np.int32)).cuda() if qstart is not None else None
    tq, tk, tv, tg = to_dev(q), to_dev(k), to_dev(v), to_dev(g)
    o, lse = ta.attn_fwd(tq, tk, tv, causal=causal, scale=float(scale), seqlens_k=sl, q_start=qs)
    dq, dk, dv = ta.attn_bwd(tq, tk, tv, o, lse, tg, causal=causal, scale=float(scale), seqlens_k=sl, q_start=qs)
    torch.cuda.synchronize()
    return f64(dq), f64(dk), f64(dv)


def compare(q, k, v, g, scale, causal, seqlens=None, qstart=None):
    dq, dk, dv = run_bwd(q, k, v, g, scale, causal, seqlens, qstart)
    rq, rk, rv = attention_bwd(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v), bf16_bits_to_f64(g),
                               float(scale), causal, seqlens_k=seqlens, q_start=qstart)
    r = check_grads({"dq": dq, "dk": dk, "dv": dv}, {"dq": rq, "dk": rk, "dv": rv})
    print("  ", r, flush=True)
    assert r.ok, str(r)
    return dq, dk, dv


SHAPES = [
    # B, H, N_q, N_k, d, causal
    (1, 1, 1, 1, 64, False),
    (1, 2, 64, 64, 64, True),
    (1, 2, 200, 200, 128, False),     # ragged tails
    (2, 1, 129, 65, 128, False),      # one row / one key past a block
    (1, 1, 100, 300, 64, True),       # N_q < N_k
    (1, 1, 300, 77, 128, True),       # N_q > N_k
    (1, 2, 256, 256, 128, True),      # whole tiles
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{s[0]}x{s[1]}x{s[2]}x{s[3]}_d{s[4]}_{'c' if s[5] else 'n'}" for s in SHAPES])
def test_bwd_shapes(shape):
    B, H, nq, nk, d, causal = shape
    q, k, v = make_random(B, H, nq, nk, d, seed=3 * nq + nk + d)
    g = make_dout((B, H, nq, d), seed=nq + 5 * nk)
    compare(q, k, v, g, np.float32(d ** -0.5), causal)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_varlen_and_masked_rows(d, causal):
    B, H, n = 4, 2, 200
    q, k, v = make_random(B, H, n, n, d, seed=200 + d)
    g = make_dout((B, H, n, d), seed=300 + d)
    seqlens = np.array([0, 63, 150, 200], np.int32)
    qstart = np.array([0, 64, 10, 200], np.int32)
    dq, dk, dv = compare(q, k, v, g, np.float32(d ** -0.5), causal, seqlens, qstart)
    assert np.all(dq[0] == 0) and np.all(dk[0] == 0) and np.all(dv[0] == 0)   # no keys
    assert np.all(dq[3] == 0) and np.all(dk[3] == 0) and np.all(dv[3] == 0)   # every row masked
    assert np.all(dq[1, :, :64] == 0)                                         # masked leading rows
    assert np.all(dk[2, :, 150:] == 0) and np.all(dv[2, :, 150:] == 0)        # keys past the valid length


RANGES = [
    # B, H, N_q, N_k, causal, seqlens_k, q_start (d = 128, several 256-key workgroups): each wave's
    # blocks split into a masked prefix (q_start, the causal diagonal), unmasked blocks and a masked
    # tail (ragged rows); some waves have keys past the valid length and no unmasked block at all
    (1, 2, 1000, 1000, 1, [900], [100]),
    (1, 2, 1000, 1000, 0, [777], [333]),
    (2, 1, 700, 900, 2, [900, 650], [0, 70]),
]


@pytest.mark.parametrize("case", RANGES, ids=[f"{c[0]}x{c[1]}x{c[2]}x{c[3]}_c{c[4]}" for c in RANGES])
def test_bwd_masked_and_unmasked_block_ranges(case):
    B, H, nq, nk, causal, sl, qs = case
    q, k, v = make_random(B, H, nq, nk, 128, seed=nq + 3 * nk + causal)
    g = make_dout((B, H, nq, 128), seed=nq + 7 * nk)
    compare(q, k, v, g, np.float32(128 ** -0.5), causal, np.array(sl, np.int32), np.array(qs, np.int32))


@pytest.mark.parametrize("scale", [0.0, -0.09, 0.3])
def test_bwd_scale_values(scale):
    q, k, v = make_random(1, 2, 130, 130, 128, seed=41)
    g = make_dout((1, 2, 130, 128), seed=42)
    compare(q, k, v, g, np.float32(scale), True)


def test_bwd_large_logits():
    q, k, v = make_random(1, 2, 300, 300, 128, seed=43, sigma=(4.0, 1.0, 1.0))
    g = make_dout((1, 2, 300, 128), seed=44)
    compare(q, k, v, g, np.float32(128 ** -0.5), True)


def test_bwd_every_element_written():
    import tiled_attention_16_amd as ta
    B, H, n, d = 2, 2, 150, 64
    q, k, v = make_random(B, H, n, n, d, seed=45)
    tq, tk, tv, tg = to_dev(q), to_dev(k), to_dev(v), to_dev(make_dout((B, H, n, d), seed=46))
    sl = torch.tensor([90, 150], dtype=torch.int32, device="cuda")
    o, lse = ta.attn_fwd(tq, tk, tv, causal=True, seqlens_k=sl)
    nan = lambda t: torch.full_like(t, float("nan"))  # noqa: E731
    dq, dk, dv = ta.attn_bwd(tq, tk, tv, o, lse, tg, causal=True, seqlens_k=sl, dq=nan(tq), dk=nan(tk), dv=nan(tv))
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert not torch.isnan(t).any().item()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_padding_keys_never_used(d, causal):
    # Keys at or past seqlens_k hold NaN (K) and +inf (V): every gradient must
    # be bit-identical to the run with ordinary values there. Lengths end
    # inside a 32-key block and inside a 256-key dK/dV tile; N_k spans three
    # such tiles.
    B, H, nq, nk = 2, 2, 300, 600
    q, k, v = make_random(B, H, nq, nk, d, seed=60 + d)
    g = make_dout((B, H, nq, d), seed=61 + d)
    seqlens = np.array([290, 531], np.int32)
    k2, v2 = k.copy(), v.copy()
    for b, n in enumerate(seqlens):
        k2[b, :, n:] = 0x7FC0   # NaN
        v2[b, :, n:] = 0x7F80   # +inf
    scale = np.float32(d ** -0.5)
    ref = compare(q, k, v, g, scale, causal, seqlens)
    got = run_bwd(q, k2, v2, g, scale, causal, seqlens)
    for x, y in zip(ref, got):
        np.testing.assert_array_equal(x, y)


def test_bwd_repeatable_bitwise():
    q, k, v = make_random(1, 2, 500, 500, 128, seed=47)
    g = make_dout((1, 2, 500, 128), seed=48)
    a = run_bwd(q, k, v, g, np.float32(128 ** -0.5), True)
    b = run_bwd(q, k, v, g, np.float32(128 ** -0.5), True)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("name", ["causal_n4096_d128", "varlen_n1024_d64"])
def test_bwd_full_size_heads(name):
    """The workload at full size, launched as the benchmark launches it; the
    oracle checks whole (batch, head) slices: eight heads spread over the head
    axis (headline shape), two heads of every batch (varlen shape)."""
    import tiled_attention_16_amd as ta
    w = WORKLOADS[name]
    inp = make_inputs(w)
    g = make_dout((w.B, w.H, w.N_q, w.d), seed=w.seed + 500)
    sl = torch.from_numpy(inp.seqlens_k).cuda() if inp.seqlens_k is not None else None
    qs = torch.from_numpy(inp.q_start).cuda() if inp.q_start is not None else None
    tq, tk, tv, tg = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v), to_dev(g)
    o, lse = ta.attn_fwd(tq, tk, tv, causal=w.causal, scale=float(inp.scale), seqlens_k=sl, q_start=qs)
    dq, dk, dv = ta.attn_bwd(tq, tk, tv, o, lse, tg, causal=w.causal, scale=float(inp.scale), seqlens_k=sl,
                             q_start=qs)
    torch.cuda.synchronize()
    dq, dk, dv = f64(dq), f64(dk), f64(dv)
    for t in (dq, dk, dv):
        assert np.all(np.isfinite(t))
    if w.B == 1:
        pairs = [(0, h) for h in range(0, w.H, max(1, w.H // 8))][:8] + [(0, w.H - 1)]
    else:
        pairs = [(b, (5 * b) % w.H) for b in range(w.B)] + [(b, w.H - 1 - (3 * b) % w.H) for b in range(w.B)]
    pairs = sorted(set(pairs))
    assert len(pairs) >= 8
    for b, h in pairs:
        sb = None if inp.seqlens_k is None else inp.seqlens_k[b:b + 1]
        qb = None if inp.q_start is None else inp.q_start[b:b + 1]
        rq, rk, rv = attention_bwd(bf16_bits_to_f64(inp.q[b:b + 1, h:h + 1]), bf16_bits_to_f64(inp.k[b:b + 1, h:h + 1]),
                                   bf16_bits_to_f64(inp.v[b:b + 1, h:h + 1]), bf16_bits_to_f64(g[b:b + 1, h:h + 1]),
                                   float(inp.scale), w.causal, seqlens_k=sb, q_start=qb)
        r = check_grads({"dq": dq[b:b + 1, h:h + 1], "dk": dk[b:b + 1, h:h + 1], "dv": dv[b:b + 1, h:h + 1]},
                        {"dq": rq, "dk": rk, "dv": rv})
        print(f"  {name} b={b} h={h}: {r}", flush=True)
        assert r.ok, f"{name} b={b} h={h}: {r}"


BR = [
    # B, H, N_q, N_k, d, seqlens, q_start
    (1, 2, 1, 500, 128, None, None),
    (1, 2, 100, 300, 64, None, None),
    (1, 1, 300, 77, 128, None, None),
    (2, 2, 257, 511, 128, [511, 300], [0, 40]),
]


@pytest.mark.parametrize("case", BR, ids=[f"{c[0]}x{c[1]}x{c[2]}x{c[3]}_d{c[4]}{'_var' if c[5] else ''}" for c in BR])
def test_bwd_bottom_right_causal(case):
    B, H, nq, nk, d, sl, qs = case
    q, k, v = make_random(B, H, nq, nk, d, seed=nq + 5 * nk + d)
    g = make_dout((B, H, nq, d), seed=nq + nk)
    compare(q, k, v, g, np.float32(d ** -0.5), 2, None if sl is None else np.array(sl, np.int32),
            None if qs is None else np.array(qs, np.int32))


def test_bwd_workspace_and_outputs_stay_in_bounds():
    """delta is [B, H, N_q, 2] floats; the kernels write nothing outside it or the gradients."""
    import tiled_attention_16_amd as ta
    B, H, n, d = 2, 2, 150, 128
    q, k, v = make_random(B, H, n, n, d, seed=61)
    tq, tk, tv, tg = to_dev(q), to_dev(k), to_dev(v), to_dev(make_dout((B, H, n, d), seed=62))
    o, lse = ta.attn_fwd(tq, tk, tv, causal=True)
    guard = 4096
    nd = B * H * n * 2
    dbuf = torch.full((nd + 2 * guard,), float("nan"), dtype=torch.float32, device="cuda")
    gbuf = torch.full((3 * B * H * n * d + 2 * guard,), float("nan"), dtype=torch.bfloat16, device="cuda")
    m = B * H * n * d
    dq = gbuf[guard:guard + m].view(B, H, n, d)
    dk = gbuf[guard + m:guard + 2 * m].view(B, H, n, d)
    dv = gbuf[guard + 2 * m:guard + 3 * m].view(B, H, n, d)
    ta.attn_bwd(tq, tk, tv, o, lse, tg, causal=True, dq=dq, dk=dk, dv=dv, delta=dbuf[guard:guard + nd].view(B, H, n, 2))
    torch.cuda.synchronize()
    assert torch.isnan(dbuf[:guard]).all().item() and torch.isnan(dbuf[guard + nd:]).all().item()
    assert torch.isnan(gbuf[:guard]).all().item() and torch.isnan(gbuf[guard + 3 * m:]).all().item()
    assert not torch.isnan(gbuf[guard:guard + 3 * m]).any().item()


MASKED = [
    # B, H, N_q, N_k, d, causal, mask shape (b, h), density
    (1, 2, 200, 300, 128, 0, (1, 2), 0.5),
    (2, 1, 300, 200, 64, 1, (2, 1), 0.7),
    (1, 2, 130, 700, 128, 2, (1, 1), 0.1),
]


@pytest.mark.parametrize("case", MASKED, ids=[f"{c[2]}x{c[3]}_d{c[4]}_c{c[5]}_p{c[7]}" for c in MASKED])
def test_bwd_dense_mask(case):
    import tiled_attention_16_amd as ta
    B, H, nq, nk, d, causal, (mb, mh), dens = case
    q, k, v = make_random(B, H, nq, nk, d, seed=nq + 7 * nk + d)
    g = make_dout((B, H, nq, d), seed=nq + 11 * nk)
    rng = np.random.default_rng(nq + nk)
    mask = rng.random((mb, mh, nq, nk)) < dens
    mask[0, 0, 3] = False                      # a row that sees no key
    mask[..., 7] = False                       # a key no row sees
    scale = np.float32(d ** -0.5)
    print(f"  masked bwd {case}", flush=True)
    tq, tk, tv, tg = to_dev(q), to_dev(k), to_dev(v), to_dev(g)
    tm = torch.from_numpy(mask).cuda()
    o, lse = ta.attn_fwd(tq, tk, tv, causal=causal, scale=float(scale), attn_mask=tm)
    dq, dk, dv = ta.attn_bwd(tq, tk, tv, o, lse, tg, causal=causal, scale=float(scale), attn_mask=tm)
    torch.cuda.synchronize()
    dq, dk, dv = f64(dq), f64(dk), f64(dv)
    rq, rk, rv = attention_bwd(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v), bf16_bits_to_f64(g),
                               float(scale), causal, attn_mask=mask)
    r = check_grads({"dq": dq, "dk": dk, "dv": dv}, {"dq": rq, "dk": rk, "dv": rv})
    print("  ", r, flush=True)
    assert r.ok, str(r)
    assert np.all(dk[:, :, 7] == 0) and np.all(dv[:, :, 7] == 0)
    assert np.all(dq[0, 0, 3] == 0)


SPARSE = [
    # B, H, N_q, N_k, d, causal, block-mask shape (b, h), density
    (1, 2, 300, 700, 128, 0, (1, 2), 0.5),
    (2, 1, 600, 600, 64, 1, (2, 1), 0.6),
    (1, 2, 520, 300, 128, 2, (1, 1), 0.4),
]


@pytest.mark.parametrize("case", SPARSE, ids=[f"{c[2]}x{c[3]}_d{c[4]}_c{c[5]}_p{c[7]}" for c in SPARSE])
def test_bwd_block_sparse(case):
    import tiled_attention_16_amd as ta
    from oracle import expand_block_mask
    B, H, nq, nk, d, causal, (mb, mh), dens = case
    q, k, v = make_random(B, H, nq, nk, d, seed=nq + 19 * nk + d)
    g = make_dout((B, H, nq, d), seed=nq + 23 * nk)
    rng = np.random.default_rng(nq + 29 * nk)
    bm = rng.random((mb, mh, -(-nq // 256), -(-nk // 128))) < dens
    bm[..., 1] = False                          # keys 128..255 in no kept block: dK = dV = 0
    scale = np.float32(d ** -0.5)
    print(f"  block-sparse bwd {case}", flush=True)
    tq, tk, tv, tg = to_dev(q), to_dev(k), to_dev(v), to_dev(g)
    tb = torch.from_numpy(bm).cuda()
    o, lse = ta.attn_fwd(tq, tk, tv, causal=causal, scale=float(scale), block_mask=tb)
    dq, dk, dv = ta.attn_bwd(tq, tk, tv, o, lse, tg, causal=causal, scale=float(scale), block_mask=tb)
    torch.cuda.synchronize()
    dq, dk, dv = f64(dq), f64(dk), f64(dv)
    rq, rk, rv = attention_bwd(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v), bf16_bits_to_f64(g),
                               float(scale), causal, attn_mask=expand_block_mask(bm, nq, nk, 256, 128))
    r = check_grads({"dq": dq, "dk": dk, "dv": dv}, {"dq": rq, "dk": rk, "dv": rv})
    print("  ", r, flush=True)
    assert r.ok, str(r)
    assert np.all(dk[:, :, 128:256] == 0) and np.all(dv[:, :, 128:256] == 0)


# The backward's first launches in a fresh process, every input uploaded anew
# just before them (cold caches and address translations): a rules-only causal
# d = 128 shape with ragged tails, a boolean-mask d = 64 shape and a varlen
# d = 64 shape, each compared with the oracle in a child process.
_FIRST_LAUNCH = r'''
import sys
import numpy as np
import torch
import tiled_attention_16_amd as ta
from oracle import attention_bwd, bf16_bits_to_f64, check_grads
from workloads import make_random

def to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)

def f64(t):
    return bf16_bits_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))

ok = True
for case in range(3):
    mask = sl = qs = None
    causal = 0
    if case == 0:
        B, H, n_q, n_k, d, causal = 1, 2, 600, 600, 128, 1
    elif case == 1:
        B, H, n_q, n_k, d = 2, 2, 200, 777, 64
        mask = np.random.default_rng(n_q * 3 + n_k).random((2, 1, n_q, n_k)) < 0.9
    else:
        B, H, n_q, n_k, d = 3, 2, 300, 300, 64
        sl, qs = np.array([300, 131, 257], np.int32), np.array([0, 40, 0], np.int32)
    q, k, v = make_random(B, H, n_q, n_k, d, seed=11 + case)
    g = make_random(B, H, n_q, n_k, d, seed=21 + case)[0]
    scale = d ** -0.5
    tm = torch.from_numpy(mask).cuda() if mask is not None else None
    tsl = torch.from_numpy(sl).cuda() if sl is not None else None
    tqs = torch.from_numpy(qs).cuda() if qs is not None else None
    o, lse = ta.attn_fwd(to_dev(q), to_dev(k), to_dev(v), causal=causal, scale=scale, seqlens_k=tsl, q_start=tqs,
                         attn_mask=tm)
    torch.cuda.synchronize()
    o_h, lse_h = o.cpu(), lse.cpu()
    dq, dk, dv = ta.attn_bwd(to_dev(q), to_dev(k), to_dev(v), o_h.cuda(), lse_h.cuda(), to_dev(g), causal=causal,
                             scale=scale, seqlens_k=tsl, q_start=tqs, attn_mask=tm)
    torch.cuda.synchronize()
    rq, rk, rv = attention_bwd(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v), bf16_bits_to_f64(g),
                               scale, causal, seqlens_k=sl, q_start=qs, attn_mask=mask)
    r = check_grads({"dq": f64(dq), "dk": f64(dk), "dv": f64(dv)}, {"dq": rq, "dk": rk, "dv": rv})
    print(f"case {case}: {r}", flush=True)
    ok = ok and r.ok
print("OK" if ok else "FAIL", flush=True)
sys.exit(0 if ok else 1)
'''


def test_first_launch_in_a_fresh_process():
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, PYTHONPATH=root + os.pathsep + os.environ.get("PYTHONPATH", ""))
    r = subprocess.run([sys.executable, "-u", "-c", _FIRST_LAUNCH], cwd=root, env=env, capture_output=True,
                       text=True, timeout=240)
    print(r.stdout, flush=True)
    assert r.returncode == 0 and "OK" in r.stdout, r.stdout + r.stderr[-2000:]
