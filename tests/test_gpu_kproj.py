"""GPU parity of k_matmul_ragged_paged_scale (through the C ABI) against the
CPU oracle.

Modular page "k_matmul_ragged_paged_scale": ragged hidden rows, row offsets,
fp8 weight with input/weight scales, output written into the paged cache of
layer layer_idx. Floats: |gpu - oracle| <= 1e-2 (|oracle| + 1); placement and
every untouched byte of the cache: bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_close, bf16v, dev16, dev32, dev8, devf32, host16, say
from oracle import numerics as nm

pytestmark = pytest.mark.gpu


def run_kproj(lib, k: synth.KProjInputs, **over):
    v = dict(hidden=k.hidden, weight=k.weight, input_scale=k.input_scale, weight_scale=k.weight_scale)
    v.update(over)
    blocks = dev16(k.blocks, torch.bfloat16)
    lib.k_matmul_ragged_paged_scale(dev16(v["hidden"], torch.bfloat16), dev32(k.row_offsets), dev8(v["weight"]),
                                    devf32(v["input_scale"]), devf32(v["weight_scale"]), blocks,
                                    dev32(k.cache_lengths), dev32(k.page_table), k.layer_idx)
    return host16(blocks)


def ref_kproj(k, **over):
    v = dict(hidden_bits=k.hidden, weight_codes=k.weight, input_scale=k.input_scale, weight_scale=k.weight_scale)
    v.update(over)
    return oracle.k_matmul_ragged_paged_scale(row_offsets=k.row_offsets, blocks_bits=k.blocks,
                                              cache_lengths=k.cache_lengths, page_table=k.page_table,
                                              layer_idx=k.layer_idx, **v)


def check(lib, k, what):
    say(f"[kproj] {what}: T={k.hidden.shape[0]} Kh={k.hidden.shape[1]} N={k.weight.shape[1]} "
        f"B={len(k.row_offsets) - 1} S={k.blocks.shape[3]}")
    got = run_kproj(lib, k)
    ref = ref_kproj(k)
    touched = np.zeros(ref.shape[:4], bool)
    _, page, slot = oracle.token_slots(k.row_offsets, k.cache_lengths, k.page_table, k.blocks.shape[3])
    touched[k.layer_idx, 0, page, slot] = True
    # every byte the oracle leaves alone is bit-identical
    assert np.array_equal(got[~touched], ref[~touched]), "cache bytes outside the written slots changed"
    return assert_close(bf16v(got[touched]), bf16v(ref[touched]), what=what)


def small(seed, lens, Kh=256, hkv=2, D=128, page_size=16, cache_lengths=None, layers=2, layer=1):
    cl = np.zeros(len(lens), np.uint32) if cache_lengths is None else np.array(cache_lengths, np.uint32)
    return synth.kproj_inputs(seed=seed, lens=list(lens), Kh=Kh, n_kv_heads=hkv, head_dim=D, page_size=page_size,
                              num_layers=layers, layer_idx=layer, cache_lengths=cl, max_len=max(lens))


def test_small_ragged(gpu, lib):
    check(lib, small(1, (5, 17, 3)), "tiny")
    check(lib, small(2, (100, 1, 64, 65, 0, 130), cache_lengths=(0, 3, 17, 128, 5, 250)), "ragged+history")
    check(lib, small(3, (300,), Kh=512, hkv=4, D=64, page_size=128), "one seq")
    check(lib, small(4, (1, 2, 3, 70), Kh=128, hkv=1, D=128, page_size=1, layers=1, layer=0), "page size 1")


def test_e4m3_codes_bit_exact(gpu, lib):
    """Each finite code once in column 0; unit hidden rows read the codes back exactly."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    k = small(5, (254,), Kh=256, hkv=1, D=128, page_size=256, layers=1, layer=0)
    w = np.zeros((256, 128), np.uint8)
    w[:254, 0] = codes
    h = nm.bf16_bits_of(np.eye(256)[:254])
    got = run_kproj(lib, k, hidden=h, weight=w, input_scale=np.ones((254, 2), np.float32),
                    weight_scale=np.ones((2, 1), np.float32))
    page = int(k.page_table[0, 0])
    col0 = bf16v(got[0, 0, page, :254, 0, 0])
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    assert np.array_equal(col0, ref)


def test_placement_fingerprint(gpu, lib):
    """Each written slot holds (t mod 256, t div 256) exactly; all other bytes keep the sentinel."""
    k = small(6, (40, 300, 1, 129, 0, 77), Kh=256, hkv=2, D=128, page_size=16,
              cache_lengths=(0, 5, 130, 17, 9, 1))
    T = int(k.row_offsets[-1])
    h = np.zeros((T, 256))
    h[:, 0] = np.arange(T) % 256
    h[:, 1] = np.arange(T) // 256
    w = np.zeros((256, 256), np.uint8)
    w[0, :128] = 0x38
    w[1, 128:] = 0x38
    got = run_kproj(lib, k, hidden=nm.bf16_bits_of(h), weight=w, input_scale=np.ones((T, 2), np.float32),
                    weight_scale=np.ones((2, 2), np.float32))
    ref = ref_kproj(k, hidden_bits=nm.bf16_bits_of(h), weight_codes=w, input_scale=np.ones((T, 2), np.float32),
                    weight_scale=np.ones((2, 2), np.float32))
    assert np.array_equal(got, ref)


def test_scale_factoring_bit_exact(gpu, lib):
    k = small(7, (33, 90))
    T = int(k.row_offsets[-1])
    base = run_kproj(lib, k, input_scale=np.ones((T, 2), np.float32), weight_scale=np.ones((2, 2), np.float32))
    scaled = run_kproj(lib, k, input_scale=np.full((T, 2), 0.25, np.float32), weight_scale=np.full((2, 2), 8.0, np.float32))
    sel = base != 0xFFFF
    assert np.array_equal(bf16v(scaled[sel]), 2.0 * bf16v(base[sel]))


def test_full_size_config(gpu, lib):
    """8 sequences (T=4312), hidden 4096, W [4096,1024] fp8, page size 128, layer 1 of 2."""
    k = synth.kproj_inputs()
    diag = check(lib, k, "full")
    say("  diagnostics", diag)


def test_full_size_with_history(gpu, lib):
    k = synth.kproj_inputs(seed=15, cache_lengths=np.array([0, 1, 127, 128, 129, 300, 1000, 5], np.uint32))
    check(lib, k, "full+history")


def test_determinism(gpu, lib):
    k = small(8, (200, 31))
    assert np.array_equal(run_kproj(lib, k), run_kproj(lib, k))


@pytest.mark.parametrize("i", range(3))
def test_tile_heights(gpu, lib, i):
    """48, 96 and 144-row tiles (the height follows the token count)."""
    from test_gpu_kv_cache import TILE_LENS
    check(lib, small(40 + i, TILE_LENS[1024][i], Kh=384, hkv=8, D=128, page_size=128), f"tile set {i}")


def test_long_hidden_rows(gpu, lib):
    """More than 32 scale blocks of K (input scales refilled in LDS every 32
    blocks): ragged, with history; 33, 40 and 97 blocks (one, one and three refills)."""
    check(lib, small(70, (100, 1, 64, 65, 0, 130), Kh=33 * 128, cache_lengths=(0, 3, 17, 128, 5, 250)), "Kh=4224")
    check(lib, small(71, (300, 7), Kh=40 * 128, hkv=2, D=128, page_size=16), "Kh=5120")
    check(lib, small(72, (500, 60), Kh=97 * 128, hkv=2, D=128, page_size=32), "Kh=12416")
