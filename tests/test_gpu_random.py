"""Seeded random shapes for every entry point against the fp64 oracle.

For each entry point a fixed seed draws a list of small configurations:
batch size, query and KV heads (group sizes 1 to 16), head dim, dtype, cache
capacity and valid lengths (with 1, the chunk and tile sizes and one past them
favoured), and for prefill the number of queries at the end of the keys.
Cache rows past the valid length are NaN; outputs sit between guard bands.
Each output must match the oracle within the dtype's bound (2e-5 fp32,
2e-2 bf16/f16).
"""

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import assert_close, note, tol_for
from tests.test_gpu_decode import run_batched, run_decode
from tests.test_gpu_prefill import run_prefill
from tests.test_gpu_q4 import oracle_q4, run_q4
from workloads import gen

pytestmark = pytest.mark.gpu

DTYPES = [torch.float32, torch.bfloat16, torch.float16]
GROUPS = [1, 2, 3, 4, 5, 6, 7, 8, 12, 16]
SPECIAL = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257]


def draw_len(rng, hi):
    if rng.random() < 0.4:
        return int(min(hi, rng.choice(SPECIAL)))
    return int(rng.integers(1, hi + 1))


def tensors(rng, B, Hq, Hkv, Tq, s_cap, D, dtype, n_valid):
    q = torch.from_numpy(rng.standard_normal((B, Hq, Tq, D), dtype=np.float32)).to(dtype)
    k = torch.from_numpy(rng.standard_normal((B, Hkv, s_cap, D), dtype=np.float32)).to(dtype)
    v = torch.from_numpy(rng.standard_normal((B, Hkv, s_cap, D), dtype=np.float32)).to(dtype)
    for b in range(B):
        n = int(n_valid[b]) if np.ndim(n_valid) else int(n_valid)
        k[b, :, n:] = float("nan")
        v[b, :, n:] = float("nan")
    return q, k, v


def test_random_decode(gpu_lib):
    rng = np.random.default_rng(20261)
    for case in range(40):
        G = int(rng.choice(GROUPS))
        Hkv = int(rng.choice([1, 2, 4]))
        D = int(rng.choice([64, 128]))
        dtype = DTYPES[int(rng.integers(0, 3))]
        B = int(rng.integers(1, 4))
        n = draw_len(rng, 3000)
        s_cap = n + int(rng.integers(0, 65))
        q, k, v = tensors(rng, B, G * Hkv, Hkv, 1, s_cap, D, dtype, n)
        note("random decode %d: %s B=%d Hq=%d Hkv=%d D=%d n=%d s_cap=%d" % (case, dtype, B, G * Hkv, Hkv, D, n, s_cap))
        got = run_decode(gpu_lib, q, k, v, n)
        assert_close(got, oracle.attend(q, k, v, kv_lens=n), tol_for(dtype), "case %d" % case)


def test_random_batched(gpu_lib):
    rng = np.random.default_rng(20262)
    for case in range(20):
        G = int(rng.choice(GROUPS))
        Hkv = int(rng.choice([1, 2, 4]))
        D = int(rng.choice([64, 128]))
        dtype = DTYPES[int(rng.integers(0, 3))]
        B = int(rng.integers(1, 10))
        s_cap = int(rng.integers(1, 2500))
        lens = np.array([0 if rng.random() < 0.1 else draw_len(rng, s_cap) for _ in range(B)], np.int32)
        q, k, v = tensors(rng, B, G * Hkv, Hkv, 1, s_cap, D, dtype, lens)
        note("random batched %d: %s B=%d Hq=%d Hkv=%d D=%d s_cap=%d lens=%s"
             % (case, dtype, B, G * Hkv, Hkv, D, s_cap, list(lens)))
        got = run_batched(gpu_lib, q, k, v, lens).cpu()
        assert_close(got, oracle.attend(q, k, v, kv_lens=lens), tol_for(dtype), "case %d" % case)
        for b in np.nonzero(lens == 0)[0]:
            assert torch.count_nonzero(got[b]) == 0


def test_random_prefill(gpu_lib):
    rng = np.random.default_rng(20263)
    for case in range(20):
        G = int(rng.choice(GROUPS[:8]))
        Hkv = int(rng.choice([1, 2]))
        D = int(rng.choice([64, 128]))
        dtype = [torch.bfloat16, torch.float16][int(rng.integers(0, 2))]
        B = int(rng.integers(1, 3))
        Tk = draw_len(rng, 1200)
        Tq = Tk if rng.random() < 0.4 else int(rng.integers(1, Tk + 1))
        s_cap = Tk + int(rng.integers(0, 65))
        q, k, v = tensors(rng, B, G * Hkv, Hkv, Tq, s_cap, D, dtype, Tk)
        note("random prefill %d: %s B=%d Hq=%d Hkv=%d D=%d Tq=%d Tk=%d s_cap=%d"
             % (case, dtype, B, G * Hkv, Hkv, D, Tq, Tk, s_cap))
        got = run_prefill(gpu_lib, q, k, v, Tk=Tk)
        assert_close(got, oracle.attend(q, k, v, kv_lens=Tk, causal=True), 2e-2, "case %d" % case)


def test_random_q4(gpu_lib):
    rng = np.random.default_rng(20264)

    class Cfg:
        pass

    for case in range(20):
        D = int(rng.choice([64, 128]))
        group = int(rng.choice([g for g in (32, 64, 128) if D % g == 0]))
        G = int(rng.choice(GROUPS))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        n = draw_len(rng, 3000)
        s_cap = n + int(rng.integers(0, 65))
        kc, ks, kb = gen.q4_encode(rng.standard_normal((1, Hkv, s_cap, D)).astype(np.float32), group)
        vc, vs, vb = gen.q4_encode(rng.standard_normal((1, Hkv, s_cap, D)).astype(np.float32), group)
        ks[:, :, n:] = np.nan
        vb[:, :, n:] = np.nan
        inp = {"q": torch.from_numpy(rng.standard_normal((1, G * Hkv, 1, D)).astype(np.float16)),
               "k_codes": torch.from_numpy(kc), "k_scales": torch.from_numpy(ks), "k_biases": torch.from_numpy(kb),
               "v_codes": torch.from_numpy(vc), "v_scales": torch.from_numpy(vs), "v_biases": torch.from_numpy(vb)}
        w = Cfg()
        w.group = group
        w.scale = lambda D=D: float(np.float32(1.0) / np.sqrt(np.float32(D)))
        note("random q4 %d: D=%d group=%d Hq=%d Hkv=%d n=%d s_cap=%d" % (case, D, group, G * Hkv, Hkv, n, s_cap))
        got = run_q4(gpu_lib, inp, w, n)
        assert_close(got, oracle_q4(inp, w, n), 2e-2, "case %d" % case)
