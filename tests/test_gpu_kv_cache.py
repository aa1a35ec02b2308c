"""GPU parity of the fused key/value projection (kv_matmul_ragged_paged_scale) and
of the e4m3 cache (both projection calls) through the C ABI, against the oracle.

The Modular page "k_matmul_ragged_paged_scale" writes into a collection that
holds keys and values and whose parameters carry a scale type and a
quantization granularity. Readings: the value weights are appended to the key
weights ([W_k | W_v]) and land in plane 1; an e4m3 cache keeps one f32 scale
s = amax / 448 per run of G head-dim elements and codes e4m3(x / s).

Bars:
  * every cache byte and scale that no token addresses: bit-exact;
  * bf16 cache: |gpu - oracle| <= 1e-2 (|oracle| + 1) per element;
  * e4m3 cache, products exact in fp32 (one-hot rows, power-of-two scales):
    codes and scales bit-exact;
  * e4m3 cache, general inputs (the kernel's fp32 GEMM differs from the exact
    product by rounding, so a code may sit one step from the oracle's where the
    value lies on a rounding midpoint): scales within 1e-4 relative, every code
    equal or adjacent to the oracle's, at most 1e-3 of them adjacent, and every
    dequantized value q * s within half a code step of the exact product:
    |q s - y| <= max(2^-4 |y|, 2^-10 s) + 1e-4 (|y| + s).
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_close, bf16v, dev16, dev32, dev8, devf32, host16, say
from oracle import numerics as nm

pytestmark = pytest.mark.gpu


def kv_inputs(seed, lens, cache_lengths=None, Kh=256, hkv=2, D=128, page_size=16, planes=2, cache="bf16",
              qgran=128, layers=2, layer=1, hidden="bf16"):
    cl = np.zeros(len(lens), np.uint32) if cache_lengths is None else np.array(cache_lengths, np.uint32)
    return synth.kproj_inputs(seed=seed, lens=list(lens), Kh=Kh, n_kv_heads=hkv, head_dim=D, page_size=page_size,
                              num_layers=layers, layer_idx=layer, cache_lengths=cl, max_len=max(max(lens), 1),
                              planes=planes, cache=cache, qgran=qgran, hidden=hidden)


def planes_of(k):
    return k.weight.shape[1] // (k.blocks.shape[4] * k.blocks.shape[5])


def tile_rows(T, N):
    """Row-tile height the library picks for T tokens and N columns: the tallest of
    48, 96 and 144 rows within 3 % of the best fill of the last pass over the CUs."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tn = N // 128
    eff = {}
    for bm in (48, 96, 144):
        tiles = -(-T // bm) * tn
        eff[bm] = T * tn / (-(-tiles // cus) * cus * bm)
    best = max(eff.values())
    return max(bm for bm in eff if eff[bm] >= best - 0.03)


# token lengths that select each row-tile height for N = 1024 and N = 2048
# (checked by test_tile_heights_are_covered)
TILE_LENS = {1024: [(700, 800), (1000, 2000), (687, 825, 24, 828, 481, 528, 646, 293)],
             2048: [(300, 400), (700, 800), (687, 825, 24, 828, 481, 528, 646, 293)]}


def run_gpu(lib, k, **over):
    v = dict(hidden=k.hidden, weight=k.weight, input_scale=k.input_scale, weight_scale=k.weight_scale)
    v.update(over)
    fp8 = k.scales is not None
    blocks = torch.from_numpy(k.blocks.copy()).cuda() if fp8 else dev16(k.blocks, torch.bfloat16)
    scales = devf32(k.scales) if fp8 else None
    fn = lib.kv_matmul_ragged_paged_scale if planes_of(k) == 2 else lib.k_matmul_ragged_paged_scale
    hid = dev8(v["hidden"]) if v["hidden"].dtype == np.uint8 else dev16(v["hidden"], torch.bfloat16)
    fn(hid, dev32(k.row_offsets), dev8(v["weight"]), devf32(v["input_scale"]),
       devf32(v["weight_scale"]), blocks, dev32(k.cache_lengths), dev32(k.page_table), k.layer_idx,
       kv_scales=scales, quantization_granularity=k.qgran)
    torch.cuda.synchronize()
    if fp8:
        return blocks.cpu().numpy(), scales.cpu().numpy()
    return host16(blocks), None


def run_ref(k, **over):
    v = dict(hidden_bits=k.hidden, weight_codes=k.weight, input_scale=k.input_scale, weight_scale=k.weight_scale)
    v.update(over)
    fn = oracle.kv_matmul_ragged_paged_scale if planes_of(k) == 2 else oracle.k_matmul_ragged_paged_scale
    out = fn(row_offsets=k.row_offsets, blocks_bits=k.blocks, cache_lengths=k.cache_lengths,
             page_table=k.page_table, layer_idx=k.layer_idx, scales=k.scales, quantization_granularity=k.qgran,
             **v)
    return out if k.scales is not None else (out, None)


def touched_rows(k):
    t = np.zeros(k.blocks.shape[:4], bool)
    _, page, slot = oracle.token_slots(k.row_offsets, k.cache_lengths, k.page_table, k.blocks.shape[3])
    t[k.layer_idx, :planes_of(k), page, slot] = True
    return t


def exact_rows_in_cache(k, magnitude=False, **over):
    """The exact product (or, with magnitude, the sum of its terms' magnitudes), laid
    out like the cache (NaN where no token writes)."""
    v = dict(hidden_bits=k.hidden, weight_codes=k.weight, input_scale=k.input_scale, weight_scale=k.weight_scale)
    v.update(over)
    if magnitude:   # clear the sign bits: |h| and |w| (the scales are positive)
        v["hidden_bits"] = v["hidden_bits"] & (0x7F if v["hidden_bits"].dtype == np.uint8 else 0x7FFF)
        v["weight_codes"] = v["weight_codes"] & 0x7F
    y = oracle.kproj_exact(**v)
    L, _, P, S, H, D = k.blocks.shape
    out = np.full((L, 2, P, S, H * D), np.nan)
    _, page, slot = oracle.token_slots(k.row_offsets, k.cache_lengths, k.page_table, S)
    for p in range(planes_of(k)):
        out[k.layer_idx, p, page, slot] = y[:, p * H * D:(p + 1) * H * D]
    return out


def check(lib, k, what):
    T, N = k.hidden.shape[0], k.weight.shape[1]
    say(f"[kv] {what}: T={T} Kh={k.hidden.shape[1]} cols={N} planes={planes_of(k)} "
        f"cache={'e4m3 G=%d' % k.qgran if k.scales is not None else 'bf16'} tile rows={tile_rows(T, N)}")
    got, gsc = run_gpu(lib, k)
    ref, rsc = run_ref(k)
    tw = touched_rows(k)
    assert np.array_equal(got[~tw], ref[~tw]), "cache bytes outside the written slots changed"
    if k.scales is None:
        return assert_close(bf16v(got[tw]), bf16v(ref[tw]), what=what)
    assert np.array_equal(gsc[~tw], rsc[~tw]), "scales outside the written slots changed"
    L, _, P, S, H, D = k.blocks.shape
    G = k.qgran
    s_g, s_r = gsc[tw].astype(np.float64), rsc[tw].astype(np.float64)        # [rows, H, D / G]
    q_g, q_r = got[tw].astype(np.uint8), ref[tw].astype(np.uint8)             # [rows, H, D]
    vg, vr = nm.decode_e4m3(q_g), nm.decode_e4m3(q_r)
    y = exact_rows_in_cache(k)[tw].reshape(q_g.shape)
    if k.hidden.dtype == np.uint8:
        # e4m3 x e4m3 MFMA: each 128-term block sum carries up to 2^-12 of the block's
        # magnitude sum (measured on the hardware: 7e-5), so the bound is on E = 2^-12 M
        E = 2.0 ** -12 * exact_rows_in_cache(k, magnitude=True)[tw].reshape(q_g.shape)
        e_run = E.reshape(E.shape[:-1] + (D // G, G)).max(axis=-1)
        assert np.all(np.abs(s_g - s_r) <= e_run / 448.0 * (1 + 2.0 ** -20) + 1e-6 * s_r), f"{what}: scales differ"
        s_full = np.repeat(s_g, G, axis=-1)
        bound = np.maximum(2.0 ** -4 * (np.abs(y) + E), 2.0 ** -10 * s_full) + E + 1e-6 * (np.abs(y) + s_full)
        bad = np.abs(vg * s_full - y) > bound
        assert not bad.any(), f"{what}: {int(bad.sum())} dequantized values beyond half a code step + E"
        return {"codes_differing": int((q_g != q_r).sum()), "codes": int(q_g.size)}
    assert np.all(np.abs(s_g - s_r) <= 1e-4 * s_r), f"{what}: scales differ"
    diff = q_g != q_r
    if diff.any():
        # adjacent codes only: same sign (or a zero) and one step apart in magnitude
        mg, mr = (q_g & 0x7F).astype(int), (q_r & 0x7F).astype(int)
        adjacent = (np.abs(mg - mr) == 1) & (((q_g ^ q_r) & 0x80 == 0) | (mg == 0) | (mr == 0))
        assert np.all(adjacent[diff]), f"{what}: codes more than one step from the oracle's"
        assert diff.mean() <= 1e-3, f"{what}: {diff.mean():.2e} of the codes differ"
    s_full = np.repeat(s_g, G, axis=-1)
    deq = vg * s_full
    bound = np.maximum(2.0 ** -4 * np.abs(y), 2.0 ** -10 * s_full) + 1e-4 * (np.abs(y) + s_full)
    bad = np.abs(deq - y) > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} dequantized values beyond half a code step"
    return {"codes_adjacent": int(diff.sum()), "codes": int(diff.size)}


def test_fused_bf16_ragged(gpu, lib):
    check(lib, kv_inputs(1, (5, 17, 3)), "tiny")
    check(lib, kv_inputs(2, (100, 1, 64, 65, 0, 130), cache_lengths=(0, 3, 17, 128, 5, 250)), "ragged+history")
    check(lib, kv_inputs(3, (300,), Kh=512, hkv=4, D=64, page_size=128), "one seq, 64-wide heads")
    check(lib, kv_inputs(4, (1, 2, 3, 70), Kh=128, hkv=1, D=128, page_size=1, layers=1, layer=0), "page size 1")


@pytest.mark.parametrize("qgran", [32, 64, 128])
def test_e4m3_cache_ragged(gpu, lib, qgran):
    for planes in (1, 2):
        check(lib, kv_inputs(10 + qgran, (5, 17, 3), planes=planes, cache="fp8", qgran=qgran), f"tiny p{planes}")
        check(lib, kv_inputs(11 + qgran, (100, 1, 64, 65, 0, 130), cache_lengths=(0, 3, 17, 128, 5, 250),
                             planes=planes, cache="fp8", qgran=qgran), f"ragged+history p{planes}")
    if qgran <= 64:
        check(lib, kv_inputs(12, (300,), Kh=512, hkv=4, D=64, page_size=128, cache="fp8", qgran=qgran),
              "64-wide heads")


@pytest.mark.parametrize("qgran", [32, 64, 128])
def test_e4m3_cache_exact_products_bit_exact(gpu, lib, qgran):
    """One-hot hidden rows times 2^-3, weight rows of nonzero finite codes with a
    +-448 in every run: the cache must hold the weight codes with scale 2^-3."""
    for planes in (1, 2):
        k = kv_inputs(20 + qgran, (9, 30, 1), cache_lengths=(3, 0, 200), planes=planes, cache="fp8", qgran=qgran)
        T = int(k.row_offsets[-1])
        Kh, NW = k.weight.shape
        rng = np.random.default_rng(qgran + planes)
        pool = np.array([c for c in range(256) if (c & 0x7F) not in (0x7F, 0x00)], np.uint8)
        w = rng.choice(pool, size=(Kh, NW)).astype(np.uint8)
        runs = w.reshape(Kh, NW // qgran, qgran)
        runs[:, :, rng.integers(0, qgran)] = np.where(rng.random((Kh, NW // qgran)) < 0.5, 0x7E, 0xFE)
        h = np.zeros((T, Kh))
        h[np.arange(T), (7 * np.arange(T)) % Kh] = 1.0
        over = dict(hidden=nm.bf16_bits_of(h), weight=w, input_scale=np.full((T, Kh // 128), 0.125, np.float32),
                    weight_scale=np.ones((Kh // 128, NW // 128), np.float32))
        say(f"[kv] exact e4m3: G={qgran} planes={planes}")
        got, gsc = run_gpu(lib, k, **over)
        ref, rsc = run_ref(k, hidden_bits=over["hidden"], weight_codes=w, input_scale=over["input_scale"],
                           weight_scale=over["weight_scale"])
        assert np.array_equal(got, ref), f"codes G={qgran} planes={planes}"
        assert np.array_equal(gsc, rsc), f"scales G={qgran} planes={planes}"


def test_e4m3_cache_ties_and_zero_tokens_bit_exact(gpu, lib):
    """Run max 448 (scale 1): 1 + 1/16 and 1.125 + 1/16 go to the even codes
    1.0 and 1.25; a zero token stores code 0 with scale 0."""
    k = kv_inputs(30, (2,), cache_lengths=(0,), planes=1, cache="fp8", qgran=32)
    Kh, NW = k.weight.shape
    h = np.zeros((2, Kh))
    h[0, 0], h[0, 1] = 1.0, 0.0625
    w = np.zeros((Kh, NW), np.uint8)
    w[0, :] = 0x38
    w[0, 1::2] = 0x39
    w[0, ::32] = 0x7E
    w[1, :] = 0x38
    w[1, ::32] = 0x00
    over = dict(hidden=nm.bf16_bits_of(h), weight=w, input_scale=np.ones((2, Kh // 128), np.float32),
                weight_scale=np.ones((Kh // 128, NW // 128), np.float32))
    got, gsc = run_gpu(lib, k, **over)
    ref, rsc = run_ref(k, hidden_bits=over["hidden"], weight_codes=w, input_scale=over["input_scale"],
                       weight_scale=over["weight_scale"])
    assert np.array_equal(got, ref) and np.array_equal(gsc, rsc)


def test_tile_heights_are_covered(gpu):
    for N, sets in TILE_LENS.items():
        assert sorted(tile_rows(sum(l), N) for l in sets) == [48, 96, 144], N


# every row-tile height (48, 96, 144 rows), keys and values, both caches
@pytest.mark.parametrize("i", range(3))
def test_tile_heights(gpu, lib, i):
    check(lib, kv_inputs(40 + i, TILE_LENS[2048][i], Kh=256, hkv=8, D=128, page_size=128), "bf16")
    check(lib, kv_inputs(50 + i, TILE_LENS[2048][i], Kh=384, hkv=8, D=128, page_size=16, cache="fp8", qgran=64),
          "e4m3")
    check(lib, kv_inputs(60 + i, TILE_LENS[1024][i], Kh=256, hkv=8, D=128, planes=1, page_size=128, cache="fp8",
                         qgran=128), "e4m3 keys")


def test_full_size(gpu, lib):
    """8 sequences (T = 4312), hidden 4096, [W_k | W_v] [4096, 2048] e4m3, page size 128:
    bf16 cache, then e4m3 cache with one scale per head (G = 128); every element."""
    say("  diagnostics", check(lib, synth.kproj_inputs(planes=2), "full bf16"))
    say("  diagnostics", check(lib, synth.kproj_inputs(planes=2, cache="fp8", qgran=128), "full e4m3"))
    say("  diagnostics", check(lib, synth.kproj_inputs(planes=1, cache="fp8", qgran=32, seed=15,
                                                       cache_lengths=np.array([0, 1, 127, 128, 129, 300, 1000, 5],
                                                                              np.uint32)), "full keys e4m3 history"))


def test_long_hidden(gpu, lib):
    """More than 32 scale blocks of K: the tile rows' input scales are refilled in
    LDS every 32 blocks (33 blocks: one refill with a one-block window; 65: two)."""
    check(lib, kv_inputs(70, (10, 130, 1), Kh=33 * 128, cache="fp8", qgran=128), "Kh=4224 e4m3")
    check(lib, kv_inputs(71, (77, 64, 3), Kh=65 * 128, cache_lengths=(5, 0, 200)), "Kh=8320 bf16")
    check(lib, kv_inputs(72, (200,), Kh=65 * 128, cache="fp8", qgran=32, planes=1), "Kh=8320 keys e4m3")


def test_determinism(gpu, lib):
    k = kv_inputs(80, (200, 31), cache="fp8", qgran=32)
    a, sa = run_gpu(lib, k)
    b, sb = run_gpu(lib, k)
    assert np.array_equal(a, b) and np.array_equal(sa, sb)
