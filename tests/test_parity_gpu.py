"""Parity of the HIP attention kernel with the fp64 CPU oracle (needs the GPU).

Every case calls the C-ABI entry point through the Python binding and compares
element by element with ``oracle.attention`` on the same seeded bf16 inputs:
  * small shapes (several tiles plus ragged tails): every output element;
  * the benchmark workloads at full size, launched exactly as bench.py launches
    them: every element of O and LSE, the mean-abs bar taken over the whole
    output, plus properties of the whole output (finite, fully masked rows
    exactly 0 with LSE = -inf);
  * grids whose workgroup count is a multiple of 8 (regrouped over the XCDs).
Bars: O max |d| <= 2e-2 and mean |d| <= 2e-3; LSE |d| <= 1e-3.
"""
import sys

import numpy as np
import pytest

from oracle import attention, bf16_bits_to_f64, check, merge
from workloads import HBM_PROBES, WORKLOADS, Workload, make_inputs, make_random, make_rising

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


def bits_of(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def run(q, k, v, scale, causal, seqlens=None, qstart=None, return_lse=True):
    import tiled_attention_16_amd as ta
    print(f"  launch B,H,Nq,Nk,d={q.shape[0]},{q.shape[1]},{q.shape[2]},{k.shape[2]},{q.shape[3]} "
          f"causal={causal} seqlens={seqlens is not None} q_start={qstart is not None}", flush=True)
    sl = torch.from_numpy(np.asarray(seqlens, np.int32)).cuda() if seqlens is not None else None
    qs = torch.from_numpy(np.asarray(qstart, np.int32)).cuda() if qstart is not None else None
    o, lse = ta.attn_fwd(to_dev(q), to_dev(k), to_dev(v), causal=causal, scale=float(scale), seqlens_k=sl,
                         q_start=qs, return_lse=return_lse)
    torch.cuda.synchronize()
    return bf16_bits_to_f64(bits_of(o)), (lse.cpu().numpy().astype(np.float64) if lse is not None else None)


def compare_full(q, k, v, scale, causal, seqlens=None, qstart=None):
    o, lse = run(q, k, v, scale, causal, seqlens, qstart)
    ro, rl = attention(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v), float(scale), causal,
                       seqlens_k=seqlens, q_start=qstart)
    r = check(o, ro, lse, rl)
    print("  ", r, flush=True)
    assert r.ok, str(r)
    return o, lse


# ------------------------------------------------------------------ small, full compare
def test_tiny_causal_d64_workload():
    w = WORKLOADS["tiny_causal_d64"]
    inp = make_inputs(w)
    compare_full(inp.q, inp.k, inp.v, inp.scale, True)


SHAPES = [
    # B, H, N_q, N_k, d, causal
    (1, 1, 1, 1, 64, False),
    (1, 1, 1, 1, 128, True),
    (1, 2, 200, 200, 64, True),       # ragged query and key tails
    (2, 1, 200, 200, 128, False),
    (1, 2, 129, 65, 128, False),      # one row / one key past a tile
    (1, 1, 100, 300, 64, True),       # N_q < N_k, causal top-left
    (1, 1, 300, 77, 128, True),       # N_q > N_k
    (1, 1, 384, 384, 128, True),      # three full query tiles
    (2, 3, 257, 511, 64, False),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{s[0]}x{s[1]}x{s[2]}x{s[3]}_d{s[4]}_{'c' if s[5] else 'n'}" for s in SHAPES])
def test_shapes(shape):
    B, H, nq, nk, d, causal = shape
    q, k, v = make_random(B, H, nq, nk, d, seed=nq * 7 + nk + d)
    compare_full(q, k, v, np.float32(d ** -0.5), causal)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_and_masked_rows(d, causal):
    B, H, n = 6, 2, 300
    q, k, v = make_random(B, H, n, n, d, seed=100 + d)
    seqlens = np.array([0, 1, 63, 64, 65, 300], np.int32)
    qstart = np.array([0, 0, 64, 100, 300, 5], np.int32)
    o, lse = compare_full(q, k, v, np.float32(d ** -0.5), causal, seqlens, qstart)
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))        # no keys at all
    assert np.all(o[4] == 0) and np.all(np.isneginf(lse[4]))        # every row masked


def test_out_of_range_mask_values_are_clamped():
    q, k, v = make_random(3, 1, 70, 70, 64, seed=5)
    compare_full(q, k, v, np.float32(0.125), False, np.array([-5, 1000, 70], np.int32),
                 np.array([-3, 0, 1000], np.int32))


# Non-causal launches with per-batch lengths hand out their workgroups heaviest
# batch first (batches ranked by valid keys times attending rows, one lane per
# batch, up to 64 batches; more batches take the plain order).
RANKED = [
    # B, H, N, d, seqlens (None: random with ties), q_start
    (64, 1, 70, 64, None, None),
    (65, 1, 40, 128, None, None),
    (7, 3, 600, 128, [600, 17, 600, 0, 333, 600, 17], [0, 0, 500, 0, 0, 599, 3]),
    (5, 2, 300, 64, [300, 300, 300, 300, 300], [0, 64, 0, 64, 300]),
    # heads over all batches a multiple of 8: whole heads dealt over the XCDs,
    # several tile pairs per head (4, 2 and 3)
    (4, 2, 1000, 64, [1000, 333, 700, 1], [0, 0, 100, 0]),
    (8, 4, 600, 128, None, None),
    (2, 4, 700, 64, [650, 700], [0, 70]),
]


@pytest.mark.parametrize("case", RANKED, ids=[f"B{c[0]}_H{c[1]}_N{c[2]}_d{c[3]}" for c in RANKED])
def test_heaviest_batch_first_order(case):
    # outputs pre-filled with NaN: a workgroup order that skipped or repeated
    # a (batch, head, tile pair) would leave NaN behind
    import tiled_attention_16_amd as ta
    B, H, n, d, sl, qs = case
    q, k, v = make_random(B, H, n, n, d, seed=B * 7 + n + d)
    rng = np.random.default_rng(B + n)
    seqlens = np.array(sl, np.int32) if sl is not None else rng.choice([1, n // 3, n // 2, n], size=B).astype(np.int32)
    qstart = np.array(qs, np.int32) if qs is not None else None
    out = torch.full((B, H, n, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H, n), float("nan"), dtype=torch.float32, device="cuda")
    print(f"  ranked B,H,N,d={B},{H},{n},{d}", flush=True)
    ta.attn_fwd(to_dev(q), to_dev(k), to_dev(v), causal=False, seqlens_k=torch.from_numpy(seqlens).cuda(),
                q_start=torch.from_numpy(qstart).cuda() if qstart is not None else None, out=out, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any().item() and not torch.isnan(lse).any().item()
    ro, rl = attention(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v), float(np.float32(d ** -0.5)),
                       False, seqlens_k=seqlens, q_start=qstart)
    r = check(bf16_bits_to_f64(bits_of(out)), ro, lse.cpu().numpy(), rl)
    print("  ", r, flush=True)
    assert r.ok, str(r)


def test_padding_contents_never_used():
    B, H, n, d = 2, 2, 150, 128
    q, k, v = make_random(B, H, n, n, d, seed=11)
    seqlens = np.array([90, 150], np.int32)
    k2, v2 = k.copy(), v.copy()
    k2[0, :, 90:] = 0x7FC0   # NaN
    v2[0, :, 90:] = 0x7F80   # +inf
    o1, l1 = run(q, k, v, np.float32(d ** -0.5), True, seqlens)
    o2, l2 = run(q, k2, v2, np.float32(d ** -0.5), True, seqlens)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


@pytest.mark.parametrize("scale", [0.0, -0.09, 0.5])
def test_scale_values(scale):
    q, k, v = make_random(1, 2, 130, 130, 128, seed=13)
    compare_full(q, k, v, np.float32(scale), True)


def test_large_logits_rescaling():
    # Q ~ N(0, 16): logits span hundreds of units; exercises every rescale path
    q, k, v = make_random(1, 2, 512, 512, 128, seed=17, sigma=(4.0, 1.0, 1.0))
    compare_full(q, k, v, np.float32(128 ** -0.5), True)
    compare_full(q, k, v, np.float32(128 ** -0.5), False)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_running_max_rises_block_after_block(d, causal):
    # Scores drift linearly along the keys: about half the rows of every wave
    # find a new maximum, several units above the old one, in nearly every
    # block of keys, so the running maximum is raised (and l and O rescaled)
    # many times per row while the other rows keep theirs.
    q, k, v = make_rising(1, 2, 300, 700, d, seed=29, step=0.5)
    compare_full(q, k, v, np.float32(d ** -0.5), causal)


# A workgroup owns two query tiles. When the first tile's slice count is a
# multiple of the ring depth, its last steps already copy the second tile's
# first K/V slices and load its Q rows; these shapes take that path (causal
# N = 1000 and non-causal N = 512 / varlen lengths that are multiples of 256 keys,
# masked leading rows inside the second tile) next to ones that do not.
CONT = [
    # B, H, N, d, causal, seqlens, q_start
    (1, 2, 1000, 128, True, None, None),
    (1, 2, 1000, 64, True, None, None),
    (2, 2, 512, 128, False, None, None),
    (2, 1, 768, 64, False, [512, 256], [100, 0]),
    (2, 1, 768, 128, True, [768, 700], [0, 260]),
    # the first tile sees 16 slices, the second none (q_start past its rows)
    (1, 2, 512, 128, True, [512], [300]),
]


@pytest.mark.parametrize("case", CONT, ids=[f"{c[0]}x{c[1]}x{c[2]}_d{c[3]}_{'c' if c[4] else 'n'}{'_var' if c[5] else ''}" for c in CONT])
def test_ring_continues_into_second_tile(case):
    B, H, n, d, causal, sl, qs = case
    q, k, v = make_random(B, H, n, n, d, seed=n + d + B)
    compare_full(q, k, v, np.float32(d ** -0.5), causal, None if sl is None else np.array(sl, np.int32),
                 None if qs is None else np.array(qs, np.int32))


def test_no_keys():
    import tiled_attention_16_amd as ta
    q = to_dev(make_random(1, 2, 40, 1, 64, seed=1)[0])
    e = torch.empty((1, 2, 0, 64), dtype=torch.bfloat16, device="cuda")
    o, lse = ta.attn_fwd(q, e, e)
    torch.cuda.synchronize()
    assert torch.all(o == 0).item() and torch.all(torch.isneginf(lse)).item()


def test_empty_query_is_noop():
    import tiled_attention_16_amd as ta
    q = torch.empty((2, 3, 0, 128), dtype=torch.bfloat16, device="cuda")
    k = to_dev(make_random(2, 3, 1, 5, 128, seed=2)[1])
    o, lse = ta.attn_fwd(q, k, k)
    assert o.shape == (2, 3, 0, 128) and lse.shape == (2, 3, 0)


def test_every_element_written_and_guards_untouched():
    import tiled_attention_16_amd as ta
    B, H, n, d = 2, 3, 190, 128
    q, k, v = make_random(B, H, n, n, d, seed=19)
    numel = B * H * n * d
    guard = 4096
    buf = torch.full((numel + 2 * guard,), float("nan"), dtype=torch.bfloat16, device="cuda")
    lbuf = torch.full((B * H * n + 2 * guard,), float("nan"), dtype=torch.float32, device="cuda")
    out = buf[guard:guard + numel].view(B, H, n, d)
    lse = lbuf[guard:guard + B * H * n].view(B, H, n)
    seqlens = torch.tensor([100, 190], dtype=torch.int32, device="cuda")
    qstart = torch.tensor([70, 0], dtype=torch.int32, device="cuda")
    ta.attn_fwd(to_dev(q), to_dev(k), to_dev(v), causal=True, seqlens_k=seqlens, q_start=qstart, out=out, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any().item()
    assert not torch.isnan(lse).any().item()
    assert torch.isnan(buf[:guard]).all().item() and torch.isnan(buf[guard + numel:]).all().item()
    assert torch.isnan(lbuf[:guard]).all().item() and torch.isnan(lbuf[guard + B * H * n:]).all().item()
    ro, rl = attention(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v), float(np.float32(d ** -0.5)),
                       True, seqlens_k=np.array([100, 190]), q_start=np.array([70, 0]))
    r = check(bf16_bits_to_f64(bits_of(out)), ro, lse.cpu().numpy(), rl)
    assert r.ok, str(r)


def test_without_lse_matches_with_lse():
    q, k, v = make_random(1, 2, 200, 200, 64, seed=23)
    o1, _ = run(q, k, v, np.float32(0.125), True)
    o2, l2 = run(q, k, v, np.float32(0.125), True, return_lse=False)
    assert l2 is None
    np.testing.assert_array_equal(o1, o2)


def test_repeatable_bitwise():
    q, k, v = make_random(1, 4, 1000, 1000, 128, seed=29)
    o1, l1 = run(q, k, v, np.float32(128 ** -0.5), True)
    o2, l2 = run(q, k, v, np.float32(128 ** -0.5), True)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


# ------------------------------------------------------------------ full-size workloads, every element
FULL = ["causal_n2048_d128", "causal_n4096_d128", "noncausal_n4096_d128", "varlen_n1024_d64",
        "causal_n16384_d128_stress", *HBM_PROBES]


def compare_whole(w: Workload, inp, o, lse):
    """Every element of O and LSE against the oracle, one batch at a time (to
    bound host memory); the mean-abs bar is taken over the whole output."""
    parts = []
    for b in range(w.B):
        sl = None if inp.seqlens_k is None else inp.seqlens_k[b:b + 1]
        qs = None if inp.q_start is None else inp.q_start[b:b + 1]
        ro, rl = attention(bf16_bits_to_f64(inp.q[b:b + 1]), bf16_bits_to_f64(inp.k[b:b + 1]),
                           bf16_bits_to_f64(inp.v[b:b + 1]), float(inp.scale), w.causal, seqlens_k=sl, q_start=qs,
                           row_block=2048)
        parts.append(check(o[b:b + 1], ro, lse[b:b + 1], rl, mean_bar=False))
        if not parts[-1].ok:
            print(f"  {w.name} b={b}: {parts[-1]}", flush=True)
    r = merge(parts)
    print(f"  {w.name} whole output ({w.B}x{w.H}x{w.N_q} rows): {r}", flush=True)
    return r


@pytest.mark.parametrize("name", FULL)
def test_full_size_workload_every_element(name):
    """The workload at full size, launched as bench.py launches it (one call,
    the whole grid: 256 or 512 workgroups, so the XCD regrouping of the
    workgroup order is in play); every output element is compared."""
    w: Workload = {**WORKLOADS, **HBM_PROBES}[name]
    inp = make_inputs(w)
    o, lse = run(inp.q, inp.k, inp.v, inp.scale, w.causal, inp.seqlens_k, inp.q_start)
    r = compare_whole(w, inp, o, lse)
    assert r.ok, f"{name}: {r}"
    if inp.q_start is not None:
        for b in range(w.B):
            qs = int(inp.q_start[b])
            assert np.all(o[b, :, :qs] == 0) and np.all(np.isneginf(lse[b, :, :qs]))
            assert np.all(np.isfinite(lse[b, :, qs:]))
    else:
        assert np.all(np.isfinite(lse))


# Rules-only d = 128 launches without per-batch lengths and with more slots
# (pairs of query tiles) than the GPU has CUs run one workgroup per CU, each
# walking several slots; a tile that spans whole ring turns fetches the next
# item's first K/V slices and its Q (the next head's included) while it
# computes. Compared whole, one batch at a time.
PERSIST = [
    # B, H, N_q, N_k, causal     (slots = B*H*ceil(ceil(N_q/256)/2) causal, B*H*ceil(N_q/256) not; 256 CUs)
    (2, 150, 256, 256, 1),       # 300 one-tile slots: every tile continues into the next head's
    (2, 140, 512, 512, 0),       # 560 one-tile slots, a head's two tiles on one XCD at once
    (1, 130, 600, 768, 0),       # three one-tile slots per head, ragged rows
    (1, 130, 1024, 256, 2),      # bottom-right: a continued tile that sees no key, keyless tiles
    (1, 300, 300, 300, 1),       # ragged: no tile spans whole ring turns, no continuation
    (2, 150, 512, 512, -1),      # negative scale (Q negated per tile), causal, continued tiles
]


@pytest.mark.parametrize("case", PERSIST, ids=[f"{c[0]}x{c[1]}x{c[2]}x{c[3]}_c{c[4]}".replace("c-1", "neg_scale")
                                         for c in PERSIST])
def test_persistent_grid_every_element(case):
    B, H, nq, nk, causal = case
    d = 128
    q, k, v = make_random(B, H, nq, nk, d, seed=nq + 7 * nk + H)
    scale = np.float32(d ** -0.5)
    if causal < 0:   # a negative score factor
        causal, scale = 1, np.float32(-0.09)
    o, lse = run(q, k, v, scale, causal)
    parts = []
    for b in range(B):
        ro, rl = attention(bf16_bits_to_f64(q[b:b + 1]), bf16_bits_to_f64(k[b:b + 1]), bf16_bits_to_f64(v[b:b + 1]),
                           float(scale), causal)
        parts.append(check(o[b:b + 1], ro, lse[b:b + 1], rl, mean_bar=False))
    r = merge(parts)
    print("  ", r, flush=True)
    assert r.ok, str(r)
    if causal == 2 and nq > nk:
        dead = nq - nk
        assert np.all(o[:, :, :dead] == 0) and np.all(np.isneginf(lse[:, :, :dead]))


# Grids whose workgroup count is a multiple of 8 take the XCD regrouping of the
# workgroup order (consecutive ids go to different XCDs; each XCD is given a
# contiguous range of (head, tile pair) indices). Small enough to compare whole.
XCD = [
    # B, H, N, d, causal   (workgroups = B*H*ceil(ceil(N/256)/2))
    (1, 8, 512, 128, True),       # 8
    (1, 8, 512, 64, False),       # 8
    (2, 4, 1000, 128, True),      # 16, ragged tail
    (2, 4, 1000, 64, False),      # 16
    (3, 8, 700, 128, False),      # 48, three tiles: one workgroup pairs tile 1 with itself
    (1, 16, 1536, 64, True),      # 48
]


@pytest.mark.parametrize("case", XCD, ids=[f"{c[0]}x{c[1]}x{c[2]}_d{c[3]}_{'c' if c[4] else 'n'}" for c in XCD])
def test_xcd_regrouped_grid_every_element(case):
    B, H, n, d, causal = case
    n_wg = B * H * ((-(-n // 256) + 1) // 2)
    assert n_wg % 8 == 0
    q, k, v = make_random(B, H, n, n, d, seed=3 * n + d + B + H)
    compare_full(q, k, v, np.float32(d ** -0.5), causal)


def test_xcd_regrouped_grid_writes_exactly_its_outputs():
    # every element of O and LSE written, nothing around them, on a regrouped grid
    import tiled_attention_16_amd as ta
    B, H, n, d = 2, 4, 1000, 128
    q, k, v = make_random(B, H, n, n, d, seed=31)
    numel = B * H * n * d
    guard = 4096
    buf = torch.full((numel + 2 * guard,), float("nan"), dtype=torch.bfloat16, device="cuda")
    lbuf = torch.full((B * H * n + 2 * guard,), float("nan"), dtype=torch.float32, device="cuda")
    out = buf[guard:guard + numel].view(B, H, n, d)
    lse = lbuf[guard:guard + B * H * n].view(B, H, n)
    seqlens = torch.tensor([1000, 613], dtype=torch.int32, device="cuda")
    qstart = torch.tensor([0, 300], dtype=torch.int32, device="cuda")
    ta.attn_fwd(to_dev(q), to_dev(k), to_dev(v), causal=True, seqlens_k=seqlens, q_start=qstart, out=out, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any().item() and not torch.isnan(lse).any().item()
    assert torch.isnan(buf[:guard]).all().item() and torch.isnan(buf[guard + numel:]).all().item()
    assert torch.isnan(lbuf[:guard]).all().item() and torch.isnan(lbuf[guard + B * H * n:]).all().item()
    ro, rl = attention(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v), float(np.float32(d ** -0.5)),
                       True, seqlens_k=np.array([1000, 613]), q_start=np.array([0, 300]))
    r = check(bf16_bits_to_f64(bits_of(out)), ro, lse.cpu().numpy(), rl)
    assert r.ok, str(r)


# Bottom-right causal (causal = 2): key j visible to row i iff j <= i + N_k - N_q.
BR = [
    # B, H, N_q, N_k, d, seqlens, q_start
    (1, 2, 1, 1000, 128, None, None),        # one new query against a cache of keys
    (1, 2, 100, 300, 64, None, None),
    (1, 1, 300, 77, 128, None, None),        # rows i < 223 see no key
    (2, 2, 257, 511, 128, [511, 300], [0, 40]),
    (2, 1, 640, 1200, 64, [1000, 1200], None),
    (1, 2, 1024, 256, 128, None, None),      # tile 3 sees 8 slices, tile 0 of its pair none
]


@pytest.mark.parametrize("case", BR, ids=[f"{c[0]}x{c[1]}x{c[2]}x{c[3]}_d{c[4]}{'_var' if c[5] else ''}" for c in BR])
def test_bottom_right_causal(case):
    B, H, nq, nk, d, sl, qs = case
    q, k, v = make_random(B, H, nq, nk, d, seed=nq + 3 * nk + d)
    o, lse = compare_full(q, k, v, np.float32(d ** -0.5), 2, None if sl is None else np.array(sl, np.int32),
                          None if qs is None else np.array(qs, np.int32))
    if nq > nk and sl is None:
        dead = nq - nk
        assert np.all(o[:, :, :dead] == 0) and np.all(np.isneginf(lse[:, :, :dead]))
