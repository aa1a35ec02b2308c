"""Pins for the ragged paged K-projection oracle (Modular page
"k_matmul_ragged_paged_scale": hidden_state, input_row_offsets, weight,
input_scale, weight_scale, kv_collection, layer_idx)."""
import json
import os

import numpy as np
import torch

import oracle
from oracle import numerics as nm
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden", "kproj_worked_example.json")
SENT = 0xFFFF


def _small(seed=0, lens=(5, 17, 3), Kh=256, hkv=2, D=128, page_size=16, cache_lengths=(0, 7, 33),
           layers=2, layer=1):
    return synth.kproj_inputs(seed=seed, lens=list(lens), Kh=Kh, n_kv_heads=hkv, head_dim=D,
                              page_size=page_size, num_layers=layers, layer_idx=layer,
                              cache_lengths=np.array(cache_lengths, np.uint32), max_len=max(lens))


def _run(k: synth.KProjInputs, **over):
    args = dict(hidden_bits=k.hidden, row_offsets=k.row_offsets, weight_codes=k.weight,
                input_scale=k.input_scale, weight_scale=k.weight_scale, blocks_bits=k.blocks,
                cache_lengths=k.cache_lengths, page_table=k.page_table, layer_idx=k.layer_idx)
    args.update(over)
    return oracle.k_matmul_ragged_paged_scale(**args)


def test_worked_example_placement_from_fixture():
    g = json.load(open(GOLD))
    K = N = 128
    offs = np.array(g["row_offsets"], np.uint32)
    T = int(offs[-1])
    h = np.zeros((T, K))
    h[:, 0] = np.arange(1, T + 1)
    w = np.zeros((K, N), np.uint8)
    np.fill_diagonal(w, 0x38)
    blocks = np.full((2, 2, 4, g["page_size"], 1, 128), SENT, np.uint16)
    out = oracle.k_matmul_ragged_paged_scale(
        nm.bf16_bits_of(h), offs, w, np.full((T, 1), 0.5, np.float32), np.full((1, 1), 2.0, np.float32),
        blocks, np.array(g["cache_lengths"], np.uint32), np.array(g["page_table"], np.uint32), 1)
    touched = np.zeros(out.shape, bool)
    for p in g["placements"]:
        row = nm.decode_bf16(out[1, 0, p["page"], p["slot"], 0])
        assert row[0] == p["value0"] and np.all(row[1:] == 0)
        touched[1, 0, p["page"], p["slot"]] = True
    assert np.all(out[~touched] == SENT)


def test_e4m3_decode_through_the_op():
    """Every finite code once in column 0: a unit hidden row reads it back exactly."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)   # 254 codes
    K = 256
    w = np.zeros((K, 128), np.uint8)
    w[:254, 0] = codes
    h = np.eye(K)[:254]
    rows = oracle.kproj_rows(nm.bf16_bits_of(h), w, np.ones((254, 2), np.float32), np.ones((2, 1), np.float32))
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    assert np.array_equal(nm.decode_bf16(rows[:, 0]), ref)


def test_placement_fingerprint_and_untouched_bytes():
    """h[t][0] = t mod 256, h[t][1] = t div 256; W routes column 0 to the first half of the
    row and column 1 to the second: each written slot names its token exactly."""
    k = _small(seed=1, lens=(40, 300, 1, 129), Kh=256, hkv=2, D=128, page_size=16,
               cache_lengths=(0, 5, 130, 17))
    T = int(k.row_offsets[-1])
    h = np.zeros((T, 256))
    h[:, 0] = np.arange(T) % 256
    h[:, 1] = np.arange(T) // 256
    w = np.zeros((256, 256), np.uint8)
    w[0, :128] = 0x38
    w[1, 128:] = 0x38
    out = _run(k, hidden_bits=nm.bf16_bits_of(h), weight_codes=w,
               input_scale=np.ones((T, 2), np.float32), weight_scale=np.ones((2, 2), np.float32))
    seen = np.zeros(out.shape, bool)
    for b in range(len(k.row_offsets) - 1):
        for j in range(int(k.row_offsets[b + 1] - k.row_offsets[b])):
            t = int(k.row_offsets[b]) + j
            pos = int(k.cache_lengths[b]) + j
            page = int(k.page_table[b, pos // 16])
            slot = pos % 16
            row = nm.decode_bf16(out[1, 0, page, slot]).ravel()
            assert np.all(row[:128] == t % 256) and np.all(row[128:] == t // 256)
            seen[1, 0, page, slot] = True
    assert np.all(out[~seen] == SENT)


def test_dense_special_case():
    """One sequence, empty cache, identity page table, unit scales: a plain rounded GEMM."""
    k = _small(seed=2, lens=(50,), cache_lengths=(0,), page_size=16, layers=1, layer=0)
    k.page_table[:] = np.arange(k.page_table.size).reshape(k.page_table.shape)
    T = 50
    ones_i = np.ones((T, 2), np.float32)
    ones_w = np.ones((2, 2), np.float32)
    out = _run(k, input_scale=ones_i, weight_scale=ones_w)
    got = out[0, 0].reshape(-1, 256)[:T]
    ta = torch.from_numpy(nm.decode_bf16(k.hidden))
    tw = torch.from_numpy(nm.decode_e4m3(k.weight))
    assert np.array_equal(nm.decode_bf16(got), nm.round_to_bf16((ta @ tw).numpy()))


def test_scale_factoring_is_exact():
    k = _small(seed=3)
    T = int(k.row_offsets[-1])
    base = _run(k, input_scale=np.ones((T, 2), np.float32), weight_scale=np.ones((2, 2), np.float32))
    scaled = _run(k, input_scale=np.full((T, 2), 0.25, np.float32), weight_scale=np.full((2, 2), 8.0, np.float32))
    sel = base != SENT
    assert np.array_equal(nm.decode_bf16(scaled[sel]), 2.0 * nm.decode_bf16(base[sel]))


def test_block_scale_locality():
    k = _small(seed=4)
    ws = k.weight_scale.copy()
    ws[1, 0] = 0.0
    w0 = k.weight.copy()
    w0[128:256, 0:128] = 0
    a = _run(k, weight_scale=ws)
    w_eff = k.weight_scale.copy()
    b = _run(k, weight_codes=w0)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, _run(k))


def test_brute_force_loops():
    k = _small(seed=5, lens=(3, 4), Kh=256, hkv=2, D=128, page_size=2, cache_lengths=(1, 2))
    out = _run(k)
    h = nm.decode_bf16(k.hidden)
    w = nm.decode_e4m3(k.weight)
    for b in range(2):
        for j in range(int(k.row_offsets[b + 1] - k.row_offsets[b])):
            t = int(k.row_offsets[b]) + j
            pos = int(k.cache_lengths[b]) + j
            page, slot = int(k.page_table[b, pos // 2]), pos % 2
            got = nm.decode_bf16(out[1, 0, page, slot]).ravel()
            for n in range(0, 256, 37):
                acc = 0.0
                for kk in range(256):
                    acc += h[t, kk] * float(k.input_scale[t, kk // 128]) * w[kk, n] * float(k.weight_scale[kk // 128, n // 128])
                assert got[n] == nm.round_to_bf16(np.array([acc]))[0]


# ---------------------------------------------------------------- keys and values, e4m3 cache

def _run_kv(k: synth.KProjInputs, **over):
    args = dict(hidden_bits=k.hidden, row_offsets=k.row_offsets, weight_codes=k.weight,
                input_scale=k.input_scale, weight_scale=k.weight_scale, blocks_bits=k.blocks,
                cache_lengths=k.cache_lengths, page_table=k.page_table, layer_idx=k.layer_idx)
    if k.scales is not None:
        args.update(scales=k.scales, quantization_granularity=k.qgran)
    args.update(over)
    fn = oracle.kv_matmul_ragged_paged_scale if args["weight_codes"].shape[1] == 2 * k.blocks.shape[4] * \
        k.blocks.shape[5] else oracle.k_matmul_ragged_paged_scale
    return fn(**args)


def _small_kv(seed=0, lens=(5, 17, 3), cache_lengths=(0, 7, 33), page_size=16, planes=2, cache="bf16", qgran=128,
              Kh=256, hkv=2, D=128):
    return synth.kproj_inputs(seed=seed, lens=list(lens), Kh=Kh, n_kv_heads=hkv, head_dim=D, page_size=page_size,
                              num_layers=2, layer_idx=1, cache_lengths=np.array(cache_lengths, np.uint32),
                              max_len=max(lens), planes=planes, cache=cache, qgran=qgran)


def _slots(k):
    for b in range(len(k.row_offsets) - 1):
        for j in range(int(k.row_offsets[b + 1] - k.row_offsets[b])):
            pos = int(k.cache_lengths[b]) + j
            S = k.blocks.shape[3]
            yield int(k.row_offsets[b]) + j, int(k.page_table[b, pos // S]), pos % S


def test_kv_planes_fingerprint_and_untouched_bytes():
    """Key columns read hidden column 0 (t mod 256), value columns read column 1
    (t div 256 + 7): plane 0 and plane 1 of each slot name the token, nothing else moves."""
    k = _small_kv(seed=1, lens=(40, 300, 1, 129), cache_lengths=(0, 5, 130, 17))
    T = int(k.row_offsets[-1])
    h = np.zeros((T, 256))
    h[:, 0] = np.arange(T) % 256
    h[:, 1] = np.arange(T) // 256 + 7
    w = np.zeros((256, 512), np.uint8)
    w[0, :256] = 0x38
    w[1, 256:] = 0x38
    out = _run_kv(k, hidden_bits=nm.bf16_bits_of(h), weight_codes=w, input_scale=np.ones((T, 2), np.float32),
                  weight_scale=np.ones((2, 4), np.float32))
    seen = np.zeros(out.shape, bool)
    for t, page, slot in _slots(k):
        assert np.all(nm.decode_bf16(out[1, 0, page, slot]) == t % 256)
        assert np.all(nm.decode_bf16(out[1, 1, page, slot]) == t // 256 + 7)
        seen[1, :, page, slot] = True
    assert np.all(out[~seen] == SENT)


def test_kv_value_plane_brute_force_loops():
    k = _small_kv(seed=6, lens=(3, 4), cache_lengths=(1, 2), page_size=2)
    out = _run_kv(k)
    h = nm.decode_bf16(k.hidden)
    w = nm.decode_e4m3(k.weight)
    for t, page, slot in _slots(k):
        got = nm.decode_bf16(out[1, 1, page, slot]).ravel()
        for n in range(0, 256, 41):
            acc = 0.0
            for kk in range(256):
                acc += (h[t, kk] * float(k.input_scale[t, kk // 128]) * w[kk, 256 + n]
                        * float(k.weight_scale[kk // 128, (256 + n) // 128]))
            assert got[n] == nm.round_to_bf16(np.array([acc]))[0]


def _onehot_e4m3_case(qgran, seed=3, planes=1):
    """Hidden token t is the unit vector e_(t mod Kh) times 2^-3, unit weight scales,
    weight rows of finite nonzero codes with a +-448 in every run of qgran columns:
    each cache run then holds exactly that weight row's codes with scale 2^-3."""
    k = _small_kv(seed=seed, lens=(9, 30), cache_lengths=(3, 0), planes=planes, cache="fp8", qgran=qgran)
    T = int(k.row_offsets[-1])
    Kh, NW = k.weight.shape
    rng = np.random.default_rng(seed)
    pool = np.array([c for c in range(256) if (c & 0x7F) not in (0x7F, 0x00)], np.uint8)
    w = rng.choice(pool, size=(Kh, NW)).astype(np.uint8)
    runs = w.reshape(Kh, NW // qgran, qgran)
    runs[:, :, rng.integers(0, qgran)] = np.where(rng.random((Kh, NW // qgran)) < 0.5, 0x7E, 0xFE)
    h = np.zeros((T, Kh))
    h[np.arange(T), np.arange(T) % Kh] = 1.0
    isc = np.full((T, Kh // 128), 0.125, np.float32)
    out, sc = _run_kv(k, hidden_bits=nm.bf16_bits_of(h), weight_codes=w, input_scale=isc,
                      weight_scale=np.ones((Kh // 128, NW // 128), np.float32))
    return k, w, out, sc


def test_e4m3_cache_reproduces_exact_codes():
    for qgran in (32, 64, 128):
        k, w, out, sc = _onehot_e4m3_case(qgran)
        n = k.blocks.shape[4] * k.blocks.shape[5]
        seen = np.zeros(out.shape, bool)
        for t, page, slot in _slots(k):
            assert np.array_equal(out[1, 0, page, slot].ravel(), w[t % w.shape[0], :n]), qgran
            assert np.all(sc[1, 0, page, slot] == 0.125), qgran
            seen[1, 0, page, slot] = True
        assert np.all(out[~seen] == 0x7F) and np.all(sc[~seen[..., :sc.shape[-1]]] == -1.0)


def test_e4m3_cache_rounds_to_nearest_even_and_zero_runs():
    """Run max 448 (scale 1): 1 + 1/16 and 1.125 + 1/16 are ties that go to the
    even codes 1.0 and 1.25; an all-zero token stores code 0 with scale 0."""
    k = _small_kv(seed=2, lens=(2,), cache_lengths=(0,), planes=1, cache="fp8", qgran=32)
    Kh, NW = k.weight.shape
    h = np.zeros((2, Kh))
    h[0, 0] = 1.0
    h[0, 1] = 0.0625
    w = np.zeros((Kh, NW), np.uint8)
    w[0, :] = 0x38            # 1.0
    w[0, 1::2] = 0x39         # 1.125
    w[0, ::32] = 0x7E         # 448: one per run of 32
    w[1, :] = 0x38            # + 0.0625 everywhere ...
    w[1, ::32] = 0x00         # ... except at the 448s
    out, sc = _run_kv(k, hidden_bits=nm.bf16_bits_of(h), weight_codes=w,
                      input_scale=np.ones((2, Kh // 128), np.float32),
                      weight_scale=np.ones((Kh // 128, NW // 128), np.float32))
    (t0, p0, s0), (t1, p1, s1) = list(_slots(k))
    row = out[1, 0, p0, s0].ravel()
    expect = np.where(np.arange(NW) % 2 == 1, 0x3A, 0x38).astype(np.uint8)
    expect[::32] = 0x7E
    assert np.array_equal(row, expect)
    assert np.all(sc[1, 0, p0, s0] == 1.0)
    assert np.all(out[1, 0, p1, s1] == 0) and np.all(sc[1, 0, p1, s1] == 0.0)


def test_e4m3_coarser_runs_take_the_largest_scale():
    """s = amax / 448 is monotone in amax: a 128-run's scale is the largest of its
    four 32-run scales, and codes agree wherever both scales are equal."""
    k32 = _small_kv(seed=8, lens=(20,), cache_lengths=(0,), planes=1, cache="fp8", qgran=32)
    k128 = _small_kv(seed=8, lens=(20,), cache_lengths=(0,), planes=1, cache="fp8", qgran=128)
    o32, s32 = _run_kv(k32)
    o128, s128 = _run_kv(k128)
    for t, page, slot in _slots(k32):
        a = s32[1, 0, page, slot].reshape(-1, 4)
        assert np.array_equal(a.max(axis=1), s128[1, 0, page, slot].ravel())
        same = np.repeat(a == a.max(axis=1, keepdims=True), 32, axis=1).ravel()
        c32 = o32[1, 0, page, slot].ravel()
        c128 = o128[1, 0, page, slot].ravel()
        assert np.array_equal(c32[same], c128[same])


# ---------------------------------------------------------------- e4m3 hidden rows

def test_e4m3_hidden_codes_through_the_op():
    """Every finite code once in hidden column 0 against a unit weight: read back exactly."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    h = np.zeros((254, 256), np.uint8)
    h[:, 0] = codes
    w = np.zeros((256, 128), np.uint8)
    w[0, 0] = 0x38
    y = oracle.kproj_exact(h, w, np.ones((254, 2), np.float32), np.ones((2, 1), np.float32))
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    assert np.array_equal(y[:, 0], ref)


def test_e4m3_hidden_equals_the_bf16_path_on_the_same_values():
    """Every e4m3 value is a bf16 value: the same numbers as bf16 bits give the same cache."""
    k8 = synth.kproj_inputs(seed=9, lens=[7, 40], Kh=256, n_kv_heads=2, head_dim=128, page_size=16, max_len=40,
                            hidden="fp8")
    as_bf16 = nm.bf16_bits_of(nm.decode_e4m3(k8.hidden))
    a = _run(k8)
    b = _run(k8, hidden_bits=as_bf16)
    assert np.array_equal(a, b)
