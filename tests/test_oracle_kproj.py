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
