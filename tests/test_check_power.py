"""Power of the prefill parity check (CPU only, oracle only).

The GPU prefill kernel splits long query rows into chunks of 64-key tiles
and merges the chunks' partial results.  A mistake where chunks meet -- one
key left out or counted twice at a tile boundary -- must fail the parity
check (max-abs 2e-2 on bf16 outputs).  On plain N(0,1) inputs with the
1/sqrt(D) scale, long rows average thousands of keys and one key moves them
by less than 1e-2, so the GPU tests use inputs with a planted key on each
side of every tile boundary (workloads.gen.seam_planted: each such key
dominates one (row, head) pair that sees it).

Here the oracle's own output is perturbed exactly as such a mistake would
(key j removed from, or counted twice in, every row that sees it, with the
softmax renormalised) and the check must reject every perturbation, for
every boundary key, in a square prefill and in a query chunk at an offset.
"""

import numpy as np
import pytest

import oracle
from workloads import gen

TOL = 2e-2


def _perturbations(q, k, v, G, keys):
    O, P = oracle.attend(q, k, v, causal=True, return_probs=True)
    vv = v.double().numpy()
    for j in keys:
        pj = P[0, :, :, j][..., None]                               # [Hq, Tq, 1]
        vj = np.repeat(vv[0, :, j], G, axis=0)[:, None, :]          # [Hq, 1, D]
        dropped = (O[0] - pj * vj) / (1.0 - pj)
        doubled = (O[0] + pj * vj) / (1.0 + pj)
        yield j, np.abs(dropped - O[0]).max(), np.abs(doubled - O[0]).max()


@pytest.mark.parametrize("Tq,Tk", [(1100, 1100), (256, 1500)])
def test_check_rejects_a_key_missed_or_doubled_at_any_tile_boundary(Tq, Tk):
    Hq, Hkv, D = 14, 2, 64
    q, k, v, keys = gen.seam_planted(1, Hq, Hkv, D, Tq, Tk, "bf16", seed=5)
    seen = 0
    for j, d_drop, d_double in _perturbations(q, k, v, Hq // Hkv, keys):
        seen += 1
        assert d_drop > TOL, "dropping key %d moves the output by only %.3e" % (j, d_drop)
        assert d_double > TOL, "doubling key %d moves the output by only %.3e" % (j, d_double)
    assert seen == len(keys) and seen >= 2 * (Tk // 64) - 2


def test_planting_is_needed_for_long_rows():
    # Without planting, long causal rows hide boundary keys: on N(0,1)
    # inputs at T = 3000 (two query heads over one KV head, the 1/sqrt(D)
    # scale) some dropped boundary key moves every output by less than the
    # bound -- the reason the GPU seam tests plant their keys.
    rng = np.random.default_rng(3000)
    T, D = 3000, 64
    q = rng.standard_normal((1, 2, T, D), dtype=np.float32)
    k = rng.standard_normal((1, 1, T, D), dtype=np.float32)
    v = rng.standard_normal((1, 1, T, D), dtype=np.float32)
    import torch

    q, k, v = (torch.from_numpy(x).to(torch.bfloat16) for x in (q, k, v))
    keys = [j for t in range(1, T // 64) for j in (64 * t - 1, 64 * t)]
    hidden = [j for j, d_drop, _ in _perturbations(q, k, v, 2, keys) if d_drop <= TOL]
    assert hidden, "expected some boundary key whose loss stays under the bound on plain inputs"
