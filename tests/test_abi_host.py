"""Host-side checks of the C ABI (no GPU needed).

* libgqa.so loads and exports every function include/gqa.h declares;
* status strings and the workspace-size function behave;
* every invalid-argument path returns its status before any HIP call.
  Only invalid calls are made here (a fully valid call would launch work),
  and no pointer passed is ever dereferenced on the host.
"""

import ctypes
import os
import re

import pytest

import prefill_split_gqa_amd as gqa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("gqa.h", "gqa_bench.h")]

FAKE = ctypes.c_void_p(0x10000)      # 16-byte aligned, never dereferenced
FAKE_ODD = ctypes.c_void_p(0x10004)  # misaligned
NULL = ctypes.c_void_p(0)


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(gqa_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    return gqa.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(gqa.EXPORTED)


def test_version_and_status_strings(lib):
    assert gqa.gqa_abi_version() == 4
    for st in range(8):
        assert gqa.status_string(st)
    assert gqa.status_string(99) == "unknown status"


def test_workspace_bytes():
    n = gqa.gqa_decode_workspace_bytes(1, 28, 4, 128, 4096)
    assert n > 0 and n % 256 == 0
    # grows with the batch, depends only on the arguments
    assert gqa.gqa_decode_workspace_bytes(8, 28, 4, 128, 4096) > n
    assert gqa.gqa_decode_workspace_bytes(1, 28, 4, 128, 4096) == n
    assert gqa.gqa_decode_workspace_bytes(1, 28, 5, 128, 4096) == 0   # Hq % Hkv
    assert gqa.gqa_decode_workspace_bytes(1, 28, 4, 96, 4096) == 0    # unsupported D
    assert gqa.gqa_decode_workspace_bytes(0, 28, 4, 128, 4096) == 0


def _decode(lib, q=FAKE, k=FAKE, v=FAKE, out=FAKE, B=1, Hq=28, Hkv=4, D=128, kv_len=10, s_cap=16,
            scale=0.1, dtype=0, ws=FAKE, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = gqa.gqa_decode_workspace_bytes(max(B, 1), Hq if Hq > 0 else 1, max(Hkv, 1), 128, max(s_cap, 1))
    return lib.gqa_decode_attend(q, k, v, out, B, Hq, Hkv, D, kv_len, s_cap, ctypes.c_float(scale), dtype, ws,
                                 ws_bytes, NULL)


def test_decode_validation(lib):
    assert _decode(lib, q=NULL) == gqa.GQA_ERR_NULL
    assert _decode(lib, out=NULL) == gqa.GQA_ERR_NULL
    assert _decode(lib, Hkv=3) == gqa.GQA_ERR_SHAPE
    assert _decode(lib, B=0) == gqa.GQA_ERR_SHAPE
    assert _decode(lib, kv_len=0) == gqa.GQA_ERR_SHAPE
    assert _decode(lib, kv_len=17) == gqa.GQA_ERR_SHAPE
    assert _decode(lib, scale=float("nan")) == gqa.GQA_ERR_SHAPE
    assert _decode(lib, D=96) == gqa.GQA_ERR_UNSUPPORTED
    assert _decode(lib, dtype=7) == gqa.GQA_ERR_UNSUPPORTED
    assert _decode(lib, ws=NULL) == gqa.GQA_ERR_WORKSPACE
    assert _decode(lib, ws_bytes=16) == gqa.GQA_ERR_WORKSPACE
    assert _decode(lib, k=FAKE_ODD) == gqa.GQA_ERR_ALIGN


def test_batched_validation(lib):
    wsb = gqa.gqa_decode_workspace_bytes(2, 32, 8, 128, 64)

    def call(lens=FAKE, B=2, Hkv=8, dtype=1, ws_bytes=wsb):
        return lib.gqa_decode_attend_batched(FAKE, FAKE, FAKE, FAKE, lens, B, 32, Hkv, 128, 64,
                                             ctypes.c_float(0.1), dtype, FAKE, ws_bytes, NULL)

    assert call(lens=NULL) == gqa.GQA_ERR_NULL
    assert call(Hkv=5) == gqa.GQA_ERR_SHAPE
    assert call(ws_bytes=wsb - 1) == gqa.GQA_ERR_WORKSPACE
    assert call(lens=FAKE_ODD) == gqa.GQA_ERR_ALIGN
    assert call(dtype=3) == gqa.GQA_ERR_UNSUPPORTED


def test_prefill_validation(lib):
    wsb = gqa.gqa_prefill_workspace_bytes(1, 14, 2, 64, 8, 8)
    assert wsb > 0

    def call(q=FAKE, Hq=14, Hkv=2, D=64, Tq=8, Tk=8, s_cap=8, dtype=1, scale=0.125, ws=FAKE, ws_bytes=wsb):
        return lib.gqa_prefill_causal(q, FAKE, FAKE, FAKE, 1, Hq, Hkv, D, Tq, Tk, s_cap, ctypes.c_float(scale),
                                      dtype, ws, ws_bytes, NULL)

    assert call(q=NULL) == gqa.GQA_ERR_NULL
    assert call(Tq=9) == gqa.GQA_ERR_SHAPE        # Tq > Tk
    assert call(Tk=9) == gqa.GQA_ERR_SHAPE        # Tk > s_cap
    assert call(Tq=0) == gqa.GQA_ERR_SHAPE
    assert call(Hkv=3) == gqa.GQA_ERR_SHAPE
    assert call(scale=float("inf")) == gqa.GQA_ERR_SHAPE
    assert call(dtype=0) == gqa.GQA_ERR_UNSUPPORTED  # fp32 prefill is not provided
    assert call(D=80) == gqa.GQA_ERR_UNSUPPORTED
    assert call(ws=NULL) == gqa.GQA_ERR_WORKSPACE
    assert call(ws_bytes=wsb - 1) == gqa.GQA_ERR_WORKSPACE
    assert call(q=FAKE_ODD) == gqa.GQA_ERR_ALIGN
    assert call(ws=FAKE_ODD) == gqa.GQA_ERR_ALIGN
    assert call(Tq=131073, Tk=131073, s_cap=131073, ws_bytes=1 << 40) == gqa.GQA_ERR_SHAPE  # row-block index width


MIB16 = 16 << 20  # fixed flag region at the front of every workspace


def test_prefill_workspace_size():
    # The flag region, then one partial slot per possible chunk of every
    # split row block.  B=2, 14 heads, T=4097: row block rb (< 32) sees
    # 2(rb+1) key tiles of 64, the last one 65, 1121 tiles a head, 31388 in
    # all; a share for each of 3 workgroups per CU (768 on 256 CUs) gives
    # chunks of at most 41 tiles, so row blocks 20..32 (13 of them) are
    # split, at most 2 ways.
    slot64 = (4 * 2 * 16 * 64 + 4 * 64 * 2) * 4
    assert gqa.gqa_prefill_workspace_bytes(2, 14, 2, 64, 4097, 4097) == MIB16 + 2 * 14 * 13 * 2 * slot64
    # one key tile: nothing is split, the flag region alone
    assert gqa.gqa_prefill_workspace_bytes(1, 14, 2, 64, 8, 8) == MIB16
    # a short prompt splits into chunks of the 3-tile floor: Tq=200 of 300
    # keys gives row blocks of 4 and 5 tiles, 2 chunks each, 14 heads
    slot128 = (4 * 4 * 16 * 64 + 4 * 64 * 2) * 4
    assert gqa.gqa_prefill_workspace_bytes(1, 14, 2, 128, 200, 300) == MIB16 + 14 * 2 * 2 * slot128
    # the 256-query chunk at offset 3841: rows of 65 tiles, at most 7 chunks
    # of 10 (the cap on chunks per row block sets the floor), 2 row blocks
    assert gqa.gqa_prefill_workspace_bytes(1, 14, 2, 64, 256, 4097) == MIB16 + 14 * 2 * 7 * slot64
    # a large batch fills the GPU without splitting
    assert gqa.gqa_prefill_workspace_bytes(64, 32, 8, 128, 2048, 2048) == MIB16
    # invalid sizes give 0
    assert gqa.gqa_prefill_workspace_bytes(1, 14, 2, 64, 9, 8) == 0
    assert gqa.gqa_prefill_workspace_bytes(1, 14, 3, 64, 8, 8) == 0
    assert gqa.gqa_prefill_workspace_bytes(1, 14, 2, 80, 8, 8) == 0


def test_decode_workspace_layout():
    # 28 query heads over 4 KV heads: 4 columns of 7 heads, 64 splits of 64
    # keys at s_cap = 4096; one 128-float partial per (column, split, head)
    # after the flag region
    assert gqa.gqa_decode_workspace_bytes(1, 28, 4, 128, 4096) == MIB16 + 4 * 64 * 7 * 128 * 4
    # the (max, sum) words, 8 bytes per partial, and five control words on
    # lines of their own (640 bytes) per (request, head tile) must fit the
    # flag region less its 64-byte tail: 28 * 64 * 8 + 4 * 640 bytes a
    # request allow 992 requests
    assert gqa.gqa_decode_workspace_bytes(992, 28, 4, 128, 4096) > 0
    assert gqa.gqa_decode_workspace_bytes(993, 28, 4, 128, 4096) == 0


def test_decode_small_heads_are_one_split():
    # a KV head of at most 8192 elements per K and V is one split (no merge):
    # 14/2 heads of 64 at s_cap = 128 -> one partial slot per (column, head);
    # at 129 rows, or at 128 rows of 128, the split plan keeps several
    assert gqa.gqa_decode_workspace_bytes(1, 14, 2, 64, 128) == MIB16 + 2 * 1 * 7 * 64 * 4
    assert gqa.gqa_decode_workspace_bytes(1, 14, 2, 64, 129) > MIB16 + 2 * 1 * 7 * 64 * 4
    assert gqa.gqa_decode_workspace_bytes(1, 28, 4, 128, 128) > MIB16 + 4 * 1 * 7 * 128 * 4
    assert gqa.gqa_decode_workspace_bytes(1, 28, 4, 128, 64) == MIB16 + 4 * 1 * 7 * 128 * 4


def test_q4_validation(lib):
    wsb = gqa.gqa_decode_workspace_bytes(1, 64, 8, 128, 64)

    def call(ks=FAKE, group=64, D=128, kv_len=10, ws_bytes=wsb):
        return lib.gqa_decode_attend_q4(FAKE, FAKE, ks, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, 8, D, group, kv_len, 64,
                                        ctypes.c_float(0.1), FAKE, ws_bytes, NULL)

    assert call(ks=NULL) == gqa.GQA_ERR_NULL
    assert call(group=48) == gqa.GQA_ERR_UNSUPPORTED
    assert call(group=128, D=64) == gqa.GQA_ERR_SHAPE
    assert call(kv_len=65) == gqa.GQA_ERR_SHAPE
    assert call(ws_bytes=0) == gqa.GQA_ERR_WORKSPACE
    assert call(ks=FAKE_ODD) == gqa.GQA_ERR_ALIGN
    assert lib.gqa_dequant_q4(NULL, FAKE, FAKE, FAKE, 4, 128, 64, NULL) == gqa.GQA_ERR_NULL
    assert lib.gqa_dequant_q4(FAKE, FAKE, FAKE, FAKE, 4, 128, 48, NULL) == gqa.GQA_ERR_UNSUPPORTED
    assert lib.gqa_dequant_q4(FAKE, FAKE, FAKE, FAKE, -1, 128, 64, NULL) == gqa.GQA_ERR_SHAPE
    assert lib.gqa_dequant_q4(FAKE, FAKE, FAKE, FAKE, 4, 96, 32, NULL) == gqa.GQA_ERR_UNSUPPORTED
    assert lib.gqa_dequant_q4(FAKE, FAKE, FAKE, FAKE, 4, 64, 128, NULL) == gqa.GQA_ERR_SHAPE


def test_q4_plan_fits_the_decode_workspace(lib):
    # the 4-bit kernel's split plan aims at fewer workgroups than the dense
    # kernels' (fewer splits), so gqa_decode_workspace_bytes covers it: with
    # exactly that many bytes the call gets past the workspace check (and
    # stops at the misaligned query pointer, before any launch)
    for B in (1, 3, 8):
        for Hq, Hkv in ((64, 8), (32, 8), (28, 4), (14, 2), (16, 16)):
            for D in (64, 128):
                for s_cap in (64, 1000, 2048, 16384):
                    wsb = gqa.gqa_decode_workspace_bytes(B, Hq, Hkv, D, s_cap)
                    assert wsb > 0
                    st = lib.gqa_decode_attend_q4(FAKE_ODD, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, B, Hq, Hkv, D,
                                                  32, s_cap, s_cap, ctypes.c_float(0.1), FAKE, wsb, NULL)
                    assert st == gqa.GQA_ERR_ALIGN, (B, Hq, Hkv, D, s_cap, st)


def test_workspace_init_validation(lib):
    assert lib.gqa_workspace_init(NULL, 256, NULL) == gqa.GQA_ERR_NULL
    assert lib.gqa_workspace_init(FAKE_ODD, 256, NULL) == gqa.GQA_ERR_ALIGN


def test_read_probe_validation(lib):
    assert lib.gqa_read_probe(NULL, 256, FAKE, NULL) == gqa.GQA_ERR_NULL
    assert lib.gqa_read_probe(FAKE, 256, NULL, NULL) == gqa.GQA_ERR_NULL
    assert lib.gqa_read_probe(FAKE, 0, FAKE, NULL) == gqa.GQA_ERR_SHAPE
    assert lib.gqa_read_probe(FAKE, 100, FAKE, NULL) == gqa.GQA_ERR_SHAPE
    assert lib.gqa_read_probe(FAKE_ODD, 256, FAKE, NULL) == gqa.GQA_ERR_ALIGN
    assert lib.gqa_read_probe(FAKE, 256, FAKE_ODD, NULL) == gqa.GQA_ERR_ALIGN


def test_library_does_not_link_the_oracle():
    # the product library and the oracle share nothing
    with open(gqa.LIB_PATH, "rb") as f:
        blob = f.read()
    assert b"gqa_oracle" not in blob


def test_append_validation(lib):
    def dense(kn=FAKE, lens=FAKE, new=NULL, B=2, D=128, T=1, s_cap=64, dtype=1):
        return lib.gqa_kv_append(kn, FAKE, FAKE, FAKE, lens, new, B, 8, D, T, s_cap, dtype, NULL)

    assert dense(kn=NULL) == gqa.GQA_ERR_NULL
    assert dense(lens=NULL) == gqa.GQA_ERR_NULL
    assert dense(T=0) == gqa.GQA_ERR_SHAPE
    assert dense(B=0) == gqa.GQA_ERR_SHAPE
    assert dense(new=FAKE, lens=FAKE) == gqa.GQA_ERR_SHAPE            # new_lens may not be kv_lens
    assert dense(D=96) == gqa.GQA_ERR_UNSUPPORTED
    assert dense(dtype=7) == gqa.GQA_ERR_UNSUPPORTED
    assert dense(kn=FAKE_ODD) == gqa.GQA_ERR_ALIGN

    def q4(kn=FAKE, lens=FAKE, new=NULL, D=128, group=64, T=1, dtype=2):
        return lib.gqa_kv_append_q4(kn, FAKE, dtype, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, lens, new, 1, 8, D, group,
                                    T, 64, NULL)

    assert q4(kn=NULL) == gqa.GQA_ERR_NULL
    assert q4(T=0) == gqa.GQA_ERR_SHAPE
    assert q4(new=FAKE) == gqa.GQA_ERR_SHAPE                          # same pointer as kv_lens
    assert q4(group=48) == gqa.GQA_ERR_UNSUPPORTED
    assert q4(group=128, D=64) == gqa.GQA_ERR_SHAPE
    assert q4(dtype=9) == gqa.GQA_ERR_UNSUPPORTED
    assert q4(kn=FAKE_ODD) == gqa.GQA_ERR_ALIGN


def test_window_sinks_validation(lib):
    wsb = gqa.gqa_decode_workspace_bytes(2, 28, 4, 128, 64)

    def dec(window=0, sinks=NULL, lens=FAKE):
        return lib.gqa_decode_attend_ex(FAKE, FAKE, FAKE, FAKE, lens, 2, 28, 4, 128, 64, ctypes.c_float(0.1), 0,
                                        window, sinks, FAKE, wsb, NULL)

    assert dec(lens=NULL) == gqa.GQA_ERR_NULL
    assert dec(window=-1) == gqa.GQA_ERR_SHAPE
    assert dec(sinks=FAKE_ODD) == gqa.GQA_ERR_ALIGN
    pwb = gqa.gqa_prefill_workspace_bytes_ex(1, 14, 2, 64, 8, 8, 3)
    assert pwb >= MIB16 and gqa.gqa_prefill_workspace_bytes_ex(1, 14, 2, 64, 8, 8, -1) == 0
    assert gqa.gqa_prefill_workspace_bytes_ex(1, 14, 2, 64, 300, 300, 0) == gqa.gqa_prefill_workspace_bytes(
        1, 14, 2, 64, 300, 300)

    def pf(window=0, sinks=NULL):
        return lib.gqa_prefill_causal_ex(FAKE, FAKE, FAKE, FAKE, 1, 14, 2, 64, 8, 8, 8, ctypes.c_float(0.125), 1,
                                         window, sinks, FAKE, pwb, NULL)

    assert pf(window=-2) == gqa.GQA_ERR_SHAPE
    assert pf(sinks=FAKE_ODD) == gqa.GQA_ERR_ALIGN


def test_q4r_validation(lib):
    # residual capacity R: a positive multiple of 64
    assert gqa.gqa_decode_q4r_workspace_bytes(2, 32, 8, 128, 4096, 128) > (16 << 20)
    assert gqa.gqa_decode_q4r_workspace_bytes(2, 32, 8, 128, 4096, 100) == 0
    assert gqa.gqa_decode_q4r_workspace_bytes(2, 32, 8, 128, 4096, 0) == 0
    assert gqa.gqa_decode_q4r_workspace_bytes(2, 32, 8, 96, 4096, 128) == 0
    wsb = gqa.gqa_decode_q4r_workspace_bytes(2, 32, 8, 128, 4096, 128)

    def dec(res=FAKE, lens=FAKE, R=128, group=64, D=128, ws_bytes=wsb, ks=FAKE):
        return lib.gqa_decode_attend_q4r(FAKE, FAKE, ks, FAKE, FAKE, FAKE, FAKE, res, FAKE, FAKE, lens, 2, 32, 8, D,
                                         group, R, 4096, ctypes.c_float(0.1), FAKE, ws_bytes, NULL)

    assert dec(res=NULL) == gqa.GQA_ERR_NULL
    assert dec(lens=NULL) == gqa.GQA_ERR_NULL
    assert dec(R=96) == gqa.GQA_ERR_SHAPE
    assert dec(group=48) == gqa.GQA_ERR_UNSUPPORTED
    assert dec(group=128, D=64) == gqa.GQA_ERR_SHAPE
    assert dec(ws_bytes=wsb - 256) == gqa.GQA_ERR_WORKSPACE
    assert dec(ks=FAKE_ODD) == gqa.GQA_ERR_ALIGN
    assert dec(res=FAKE_ODD) == gqa.GQA_ERR_ALIGN

    def app(kn=FAKE, res=FAKE, lens=FAKE, new=NULL, R=128, group=64, D=128, T=1):
        return lib.gqa_kv_append_q4r(kn, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, res, FAKE, lens, new, 2, 8, D,
                                     group, R, T, 4096, NULL)

    assert app(kn=NULL) == gqa.GQA_ERR_NULL
    assert app(res=NULL) == gqa.GQA_ERR_NULL
    assert app(T=0) == gqa.GQA_ERR_SHAPE
    assert app(R=32) == gqa.GQA_ERR_SHAPE
    assert app(new=FAKE) == gqa.GQA_ERR_SHAPE                         # same pointer as kv_lens
    assert app(group=48) == gqa.GQA_ERR_UNSUPPORTED
    assert app(D=96) == gqa.GQA_ERR_UNSUPPORTED
    assert app(res=FAKE_ODD) == gqa.GQA_ERR_ALIGN

    wsp = gqa.gqa_prefill_workspace_bytes(1, 14, 2, 64, 256, 4097)

    def pf(res=FAKE, R=128, group=32, D=64, Tq=256, Tk=4097, s_cap=4097, ws_bytes=wsp, out=FAKE):
        return lib.gqa_prefill_causal_q4r(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, res, FAKE, out, 1, 14, 2, D, group,
                                          R, Tq, Tk, s_cap, ctypes.c_float(0.125), FAKE, ws_bytes, NULL)

    assert pf(res=NULL) == gqa.GQA_ERR_NULL
    assert pf(out=NULL) == gqa.GQA_ERR_NULL
    assert pf(Tq=4098) == gqa.GQA_ERR_SHAPE
    assert pf(s_cap=4000) == gqa.GQA_ERR_SHAPE
    assert pf(R=100) == gqa.GQA_ERR_SHAPE
    assert pf(group=128) == gqa.GQA_ERR_SHAPE                         # group larger than D
    assert pf(group=16) == gqa.GQA_ERR_UNSUPPORTED
    assert pf(D=96) == gqa.GQA_ERR_UNSUPPORTED
    assert pf(ws_bytes=0) == gqa.GQA_ERR_WORKSPACE
    assert pf(res=FAKE_ODD) == gqa.GQA_ERR_ALIGN
