"""Small helpers shared by the GPU parity tests (comparison and guard bands)."""

import sys

import numpy as np
import torch

TOL_F32 = 2e-5   # max-abs bound for fp32 outputs
TOL_16 = 2e-2    # max-abs bound for bf16 / f16 outputs


def tol_for(dtype) -> float:
    return TOL_F32 if dtype == torch.float32 else TOL_16


def note(msg: str) -> None:
    """Flush a line naming the case before a GPU step (survives a crash)."""
    sys.stdout.write(msg + "\n")
    sys.stdout.flush()


def max_abs_err(got: torch.Tensor, want: np.ndarray) -> float:
    g = got.detach().float().cpu().double().numpy()
    assert g.shape == want.shape, (g.shape, want.shape)
    assert np.isfinite(g).all(), "non-finite output"
    return float(np.abs(g - want).max()) if g.size else 0.0


def row_ulps(got: torch.Tensor, want: np.ndarray) -> np.ndarray:
    """Per output row (last axis), the max-abs error in units in the last
    place of the output dtype at the row's largest |oracle value|
    (bf16: 8 significant bits, f16: 11, fp32: 24)."""
    bits = {torch.bfloat16: 8, torch.float16: 11, torch.float32: 24}[got.dtype]
    g = got.detach().float().cpu().double().numpy()
    err = np.abs(g - want).max(axis=-1)
    top = np.maximum(np.abs(want).max(axis=-1), 2.0 ** -126)
    ulp = np.exp2(np.floor(np.log2(top)) - (bits - 1))
    return err / ulp


def assert_close(got: torch.Tensor, want: np.ndarray, tol: float, what: str, max_ulps=None) -> float:
    err = max_abs_err(got, want)
    if got.dtype in (torch.bfloat16, torch.float16) and got.numel():
        u = row_ulps(got, want)
        note("  %s: max-abs error %.3e (bound %.1e); per-row error up to %.2f ulps of the row max%s"
             % (what, err, tol, float(u.max()), "" if max_ulps is None else " (bound %g)" % max_ulps))
        if max_ulps is not None:
            assert float(u.max()) <= max_ulps, "%s: %.2f ulps > %g" % (what, float(u.max()), max_ulps)
    else:
        note("  %s: max-abs error %.3e (bound %.1e)" % (what, err, tol))
    assert err <= tol, "%s: max-abs error %.3e > %.1e" % (what, err, tol)
    return err


class Guarded:
    """An output tensor with sentinel-filled guard bands on both sides."""

    PAD = 256  # elements (keeps 16-byte alignment for every dtype used)

    def __init__(self, shape, dtype, device="cuda", sentinel=1234.5):
        n = int(np.prod(shape))
        self.buf = torch.full((n + 2 * self.PAD,), sentinel, dtype=dtype, device=device)
        self.sentinel = sentinel
        self.n = n
        self.t = self.buf[self.PAD:self.PAD + n].view(*shape)

    def check(self):
        b = self.buf.float().cpu()
        s = torch.tensor(self.sentinel, dtype=self.buf.dtype).float()
        assert (b[:self.PAD] == s).all() and (b[self.PAD + self.n:] == s).all(), "write outside the output"


REGION_BYTES = 16 << 20  # region at the front of every workspace


def assert_workspace_ready(ws: torch.Tensor, what: str) -> None:
    """A workspace between calls: the 16 MiB region zero-filled, and every
    32-bit word after it with its lowest bit clear (decode recognises its
    published partial words by that bit)."""
    torch.cuda.synchronize()
    head = ws[:REGION_BYTES]
    assert int((head != 0).sum()) == 0, "region not zero-filled: " + what
    rest = ws[REGION_BYTES:]
    n = rest.numel() // 4 * 4
    words = rest[:n].view(torch.int32)
    assert int((words & 1).sum()) == 0, "a word past the region has its lowest bit set: " + what
