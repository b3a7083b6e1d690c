"""The C ABI on the host (no GPU needed): the library loads, exports every function
include/g4attn.h declares, the ctypes mirrors match the C structs, and every
fail-closed path returns its status before any HIP call (nothing is launched)."""
import ctypes
import os
import re

import pytest

import global_gqa_attention_amd as g
import workloads as W

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "g4attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(g.LIB_PATH), reason="libg4attn.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(g4attn_\w+)\s*\(", src)))


def test_exports_every_declared_function():
    names = declared_functions()
    assert set(names) == set(g.EXPORTED), names
    L = g.lib()
    for n in names:
        assert hasattr(L, n), n


def test_abi_version():
    assert g.g4attn_abi_version() == 3


def test_struct_layouts():
    assert ctypes.sizeof(g.Layer) == 56
    assert g.Layer.rope_theta.offset == 40
    assert ctypes.sizeof(g.Provenance) == 64 + 12 * 4 + 8


def _layer(spec=W.SLIDING_31B, **over):
    L = g.make_layer(spec)
    for k, v in over.items():
        setattr(L, k, v)
    return L


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def _prefill(layer, q=FAKE, k=FAKE, v=FAKE, out=FAKE, ss=FAKE, sl=FAKE, batch=1, maxlen=16):
    return g.lib().g4attn_prefill(ctypes.byref(layer), q, k, v, out, ss, sl, batch, maxlen, None, None)


def _decode(layer, q=FAKE, kc=FAKE, vc=FAKE, row0=FAKE, ctx=FAKE, slots=1024, out=FAKE, batch=1, maxctx=100):
    return g.lib().g4attn_decode(ctypes.byref(layer), q, kc, vc, row0, ctx, slots, out, batch, maxctx, None, None,
                                 None)


def _prologue(layer, q=FAKE, k=FAKE, v=None, vo=None, wq=FAKE, wk=FAKE, pos=FAKE, dst=None, n=4):
    return g.lib().g4attn_qk_prologue(ctypes.byref(layer), q, q, k, k, v, vo, wq, wk, pos, dst, n, None)


INVALID, UNSUPPORTED = g.G4ATTN_ERR_INVALID_ARG, g.G4ATTN_ERR_UNSUPPORTED


@pytest.mark.parametrize("over,code", [
    (dict(num_q_heads=30), INVALID),          # Hq % Hkv != 0
    (dict(num_kv_heads=0), INVALID),
    (dict(num_q_heads=48, num_kv_heads=1), UNSUPPORTED),  # G = 48
    (dict(num_q_heads=12, num_kv_heads=4), UNSUPPORTED),  # G = 3
    (dict(head_dim=96), UNSUPPORTED),
    (dict(head_dim=1024), UNSUPPORTED),
    (dict(window=-1), INVALID),
    (dict(window=0), INVALID),                # sliding kind needs a window
    (dict(kind=7), INVALID),
    (dict(v_norm=2), INVALID),
    (dict(v_norm=1, k_eq_v=1), INVALID),     # the value norm needs a separate V
    (dict(k_eq_v=2), INVALID),
    (dict(softmax_scale=0.0), INVALID),
    (dict(softmax_scale=float("nan")), INVALID),
    (dict(rms_eps=-1.0), INVALID),
    (dict(rope_dims=255), INVALID),           # odd
    (dict(rope_dims=512), INVALID),           # > D
    (dict(rope_freq_dim=0), INVALID),
    (dict(rope_theta=0.0), INVALID),
    (dict(rope_pairing=5), INVALID),
    (dict(rope_dims=12), UNSUPPORTED),        # R/2 = 6 not a multiple of 8
])
def test_layer_validation_fails_closed(over, code):
    L = _layer(**over)
    assert _prefill(L) == code
    assert g.g4attn_last_error() != ""
    assert _decode(L) == code
    assert _prologue(L) == code


def test_global_kind_needs_full_causal():
    assert _prefill(_layer(W.GLOBAL_31B, window=1024), v=None) == INVALID


def test_prefill_argument_checks():
    L = _layer()
    assert _prefill(L, q=None) == INVALID
    assert _prefill(L, out=None) == INVALID
    assert _prefill(L, v=None) == INVALID                       # separate V missing
    assert _prefill(_layer(W.GLOBAL_31B), v=FAKE) == INVALID    # V given for K=V
    assert _prefill(L, batch=-1) == INVALID
    assert _prefill(L, maxlen=-5) == INVALID
    assert _prefill(L, ss=None) == INVALID
    # head dim 512 with separate K and V (the real model's global layer) passes validation
    assert _prefill(_layer(W.GLOBAL_31B, k_eq_v=0, v_norm=1), v=FAKE, batch=0) == g.G4ATTN_OK
    # a long sequence passes validation (no span limit; empty batch, so nothing launches)
    assert _prefill(L, batch=0, maxlen=1 << 30) == g.G4ATTN_OK
    # out must be a buffer of its own (checked last, before any launch)
    for alias in ("q", "k", "v"):
        args = dict(q=FAKE + 0x100, k=FAKE + 0x200, v=FAKE + 0x300, out=FAKE)
        args[alias] = FAKE
        assert _prefill(L, **args) == INVALID, alias
        assert "out" in g.g4attn_last_error()
    # empty work is OK and launches nothing
    assert _prefill(L, batch=0) == g.G4ATTN_OK and g.g4attn_last_error() == ""
    assert _prefill(L, maxlen=0) == g.G4ATTN_OK


def test_decode_argument_checks():
    L = _layer()
    assert _decode(L, slots=1000) == INVALID                    # ring smaller than the window
    assert _decode(L, slots=0) == INVALID
    assert _decode(L, row0=None) == INVALID
    assert _decode(L, maxctx=0) == INVALID
    Lg = _layer(W.GLOBAL_31B)
    assert _decode(Lg, vc=None, slots=100, maxctx=101) == INVALID  # linear cache too short
    assert _decode(Lg, vc=FAKE, slots=200, maxctx=100) == INVALID  # V given for K=V
    assert _decode(Lg, vc=None, slots=1 << 20, maxctx=100) == UNSUPPORTED  # > 2 GiB span
    assert _decode(L, batch=0) == g.G4ATTN_OK


def _cached(layer, q=FAKE, kc=FAKE, vc=FAKE, out=FAKE, qr=FAKE, qp=FAKE, cl=FAKE, row0=FAKE, slots=1536, batch=1,
            maxchunk=512, maxkey=4096):
    return g.lib().g4attn_prefill_cached(ctypes.byref(layer), q, kc, vc, out, qr, qp, cl, row0, slots, batch, maxchunk,
                                         maxkey, None, None)


def test_prefill_cached_argument_checks():
    # every call below fails validation (or is empty work), so the FAKE pointers are never used
    L = _layer()
    assert _cached(L, slots=1535) == INVALID                    # not a multiple of 32
    assert g.g4attn_last_error() != ""
    assert _cached(L, slots=1504) == INVALID                    # ring < window + chunk
    assert _cached(L, slots=0) == INVALID
    assert _cached(L, q=None) == INVALID
    assert _cached(L, vc=None) == INVALID                       # separate V missing
    assert _cached(L, qp=None) == INVALID
    assert _cached(L, row0=None) == INVALID
    assert _cached(L, batch=-1) == INVALID
    assert _cached(L, maxkey=100) == INVALID                    # fewer keys than chunk rows
    Lg = _layer(W.GLOBAL_31B)
    assert _cached(Lg, vc=None, slots=1024, maxkey=2048) == INVALID  # linear cache too short
    assert _cached(Lg, vc=FAKE, slots=4096, maxkey=2048) == INVALID  # V given for K=V
    assert _cached(_layer(W.GLOBAL_31B, k_eq_v=0), vc=FAKE, slots=4096, maxkey=2048, batch=0) == g.G4ATTN_OK
    for alias in ("q", "kc", "vc"):
        args = dict(q=FAKE + 0x100, kc=FAKE + 0x200, vc=FAKE + 0x300, out=FAKE)
        args[alias] = FAKE
        assert _cached(L, **args) == INVALID, alias
    assert _cached(L, batch=0) == g.G4ATTN_OK and g.g4attn_last_error() == ""
    assert _cached(L, maxchunk=0) == g.G4ATTN_OK


def _masked(layer, q=FAKE, k=FAKE, v=FAKE, out=FAKE, st=FAKE, ln=FAKE, lk=FAKE, batch=1, maxlen=64):
    return g.lib().g4attn_prefill_masked(ctypes.byref(layer), q, k, v, out, st, ln, lk, batch, maxlen, None, None)


def test_prefill_masked_argument_checks():
    # every call below fails validation (or is empty work), so the FAKE pointers are never used
    L = _layer()
    assert _masked(L, lk=None) == INVALID                       # last keys missing
    assert g.g4attn_last_error() != ""
    assert _masked(L, q=None) == INVALID
    assert _masked(L, v=None) == INVALID                        # separate V missing
    assert _masked(L, st=None) == INVALID
    assert _masked(L, batch=-1) == INVALID
    assert _masked(L, maxlen=-1) == INVALID
    assert _masked(_layer(W.GLOBAL_31B), v=FAKE) == INVALID     # V given for K=V
    assert _masked(_layer(W.GLOBAL_31B, k_eq_v=0), batch=0) == g.G4ATTN_OK
    assert _masked(L, lk=None, batch=0) == g.G4ATTN_OK and g.g4attn_last_error() == ""
    assert _masked(L, maxlen=0) == g.G4ATTN_OK


def test_prefill_cached_masked_argument_checks():
    # every call below fails validation (or is empty work), so the FAKE pointers are never used
    L = _layer()
    lib = g.lib()

    def call(lk=FAKE, slots=1536, batch=1, maxchunk=512):
        return lib.g4attn_prefill_cached_masked(ctypes.byref(L), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, lk, FAKE,
                                                slots, batch, maxchunk, 4096, None, None)

    assert call(lk=None) == INVALID                              # last keys missing
    assert call(slots=1535) == INVALID                           # the cached checks still apply
    assert call(batch=-1) == INVALID
    assert call(lk=None, batch=0) == g.G4ATTN_OK
    assert call(maxchunk=0) == g.G4ATTN_OK


def test_prologue_argument_checks():
    L = _layer()
    lib = g.lib()
    assert lib.g4attn_qk_prologue(ctypes.byref(L), FAKE, None, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, None, 4,
                                  None) == INVALID            # q_out missing
    assert _prologue(L, q=None, k=None) == INVALID            # nothing to do
    assert _prologue(L, wq=None) == INVALID
    assert _prologue(L, pos=None) == INVALID
    assert _prologue(L, n=-1) == INVALID
    assert _prologue(_layer(W.GLOBAL_31B), v=FAKE, vo=FAKE + 64) == INVALID  # V for K=V
    assert _prologue(L, dst=FAKE) == INVALID                  # scatter in place
    assert _prologue(L, n=0) == g.G4ATTN_OK


def test_prefill_backward_argument_checks():
    L, Lg = _layer(), _layer(W.GLOBAL_31B)
    lib = g.lib()

    def call(layer=L, q=FAKE, k=FAKE + 8, v=FAKE + 16, out=FAKE + 24, do=FAKE + 32, dq=FAKE + 40, dk=FAKE + 48,
             dv=FAKE + 56, lse=FAKE + 64, delta=FAKE + 72, batch=1, maxlen=64):
        return lib.g4attn_prefill_backward(ctypes.byref(layer), q, k, v, out, do, dq, dk, dv, lse, delta, FAKE, FAKE,
                                           batch, maxlen, None)

    assert call(q=None) == INVALID
    assert call(lse=None) == INVALID
    assert call(v=None) == INVALID                          # separate V missing
    assert call(dv=None) == INVALID
    assert call(layer=Lg) == INVALID                        # v / dv given for K=V
    assert call(dq=FAKE) == INVALID                          # an output aliasing an input
    assert call(dk=FAKE + 24) == INVALID
    assert call(batch=-1) == INVALID
    assert call(layer=_layer(head_dim=96)) == UNSUPPORTED
    assert call(batch=0) == g.G4ATTN_OK and g.g4attn_last_error() == ""
    assert call(layer=Lg, v=None, dv=None, batch=0) == g.G4ATTN_OK


def _split_bytes(layer, batch, rows, maxkey, keys):
    n = ctypes.c_uint64(123)
    st = g.lib().g4attn_split_workspace_bytes(ctypes.byref(layer), batch, rows, maxkey, keys, ctypes.byref(n))
    return st, n.value


def test_split_workspace_bytes():
    Lg = _layer(W.GLOBAL_31B)
    Hq, D = Lg.num_q_heads, Lg.head_dim
    # prefill of 2 x 1000 rows at chunks of 256: 4 chunk slots per row, D + 2 floats each
    assert _split_bytes(Lg, 2, 1000, 1000, 256) == (g.G4ATTN_OK, 2 * 1000 * Hq * 4 * (D + 2) * 4)
    # decode of 64 rows up to 32768 keys at chunks of 4096: 8 chunk slots
    assert _split_bytes(Lg, 64, 1, 32768, 4096) == (g.G4ATTN_OK, 64 * Hq * 8 * (D + 2) * 4)
    # no row spans two chunks: nothing to hold
    assert _split_bytes(Lg, 4, 1, 4096, 4096) == (g.G4ATTN_OK, 0)
    assert _split_bytes(Lg, 0, 1, 9000, 4096) == (g.G4ATTN_OK, 0)
    assert _split_bytes(Lg, 4, 1, 4097, 4096)[1] == 4 * Hq * 2 * (D + 2) * 4
    # chunk sizes: positive multiples of 256; global layers only
    assert _split_bytes(Lg, 1, 1, 100, 0)[0] == INVALID
    assert _split_bytes(Lg, 1, 1, 100, 300)[0] == INVALID
    assert _split_bytes(Lg, 1, 1, 100, -256)[0] == INVALID
    assert _split_bytes(_layer(), 1, 1, 100, 256)[0] == UNSUPPORTED
    assert "global" in g.g4attn_last_error()
    assert _split_bytes(Lg, -1, 1, 100, 256)[0] == INVALID
    assert g.lib().g4attn_split_workspace_bytes(ctypes.byref(Lg), 1, 1, 100, 256, None) == INVALID


def _prefill_split(layer, q=FAKE, k=FAKE, v=None, out=FAKE + 0x40, ss=FAKE, sl=FAKE, batch=1, maxlen=1000,
                   keys=256, ws=FAKE + 0x800, wsb=1 << 40):
    return g.lib().g4attn_prefill_split(ctypes.byref(layer), q, k, v, out, ss, sl, batch, maxlen, keys, ws, wsb, None,
                                        None)


def _decode_split(layer, q=FAKE, kc=FAKE, row0=FAKE, ctx=FAKE, slots=40000, out=FAKE + 0x40, batch=4,
                  maxctx=32768, keys=4096, ws=FAKE + 0x800, wsb=1 << 40):
    return g.lib().g4attn_decode_split(ctypes.byref(layer), q, kc, None, row0, ctx, slots, out, batch, maxctx, None,
                                       keys, ws, wsb, None, None)


def test_split_argument_checks():
    # every call below fails validation (or is empty work), so the FAKE pointers are never used
    Lg = _layer(W.GLOBAL_31B)
    need = _split_bytes(Lg, 1, 1000, 1000, 256)[1]
    assert _prefill_split(Lg, keys=100) == INVALID
    assert _prefill_split(_layer(), v=FAKE) == UNSUPPORTED          # sliding layer
    assert _prefill_split(Lg, ws=None) == INVALID                    # workspace needed
    assert "workspace" in g.g4attn_last_error()
    assert _prefill_split(Lg, wsb=need - 1) == INVALID               # too small
    assert _prefill_split(Lg, ws=FAKE + 0x808) == INVALID            # not 16-byte aligned
    assert _prefill_split(Lg, ws=FAKE) == INVALID                    # the workspace is q
    assert _prefill_split(Lg, out=FAKE) == INVALID                   # out is q
    assert _prefill_split(Lg, batch=0) == g.G4ATTN_OK
    assert _prefill_split(Lg, maxlen=0, ws=None) == g.G4ATTN_OK
    need_d = _split_bytes(Lg, 4, 1, 32768, 4096)[1]
    assert _decode_split(Lg, keys=512 + 1) == INVALID
    assert _decode_split(Lg, ws=None) == INVALID
    assert _decode_split(Lg, wsb=need_d - 16) == INVALID
    assert _decode_split(Lg, slots=1000) == INVALID                  # linear cache too short
    assert _decode_split(Lg, out=FAKE) == INVALID
    assert _decode_split(Lg, batch=0) == g.G4ATTN_OK
    assert _decode_split(_layer(), keys=4096) == UNSUPPORTED


def test_split_noalloc_rejects_requests_beyond_its_array():
    # every call below fails validation (or is empty work), so the FAKE pointers are never used
    Lg = _layer(W.GLOBAL_31B)

    def call(batch, maxctx, keys):
        return g.lib().g4attn_decode_split_noalloc(ctypes.byref(Lg), FAKE, FAKE, None, FAKE, FAKE, 40000, FAKE + 0x40,
                                                   batch, maxctx, None, keys, None, None)

    # 256 sequences of up to 32768 keys in chunks of 256: 2 GiB of partial results > 64 MiB
    assert call(256, 32768, 256) == UNSUPPORTED
    assert "scratch" in g.g4attn_last_error()
    assert call(4, 1000, 300) == INVALID          # chunk size not a multiple of 256
    assert call(0, 32768, 4096) == g.G4ATTN_OK    # nothing to do
    assert call(-1, 32768, 4096) == INVALID


def _prefill_qp(layer, q=FAKE, w=FAKE + 0x10, pos=FAKE + 0x20, k=FAKE + 0x30, v=None, out=FAKE + 0x40, ss=FAKE,
                sl=FAKE, batch=1, maxlen=16):
    return g.lib().g4attn_prefill_qp(ctypes.byref(layer), q, w, pos, k, v, out, ss, sl, batch, maxlen, None, None)


def test_prefill_qp_argument_checks():
    G = _layer(W.GLOBAL_31B)
    assert _prefill_qp(G, w=None) == INVALID
    assert _prefill_qp(G, pos=None) == INVALID
    assert _prefill_qp(G, q=None) == INVALID
    assert _prefill_qp(G, out=FAKE) == INVALID                         # out aliases q
    # head dim 512 with K=V only
    assert _prefill_qp(_layer(), v=FAKE + 0x50) == UNSUPPORTED      # sliding layer
    assert _prefill_qp(_layer(W.GLOBAL_31B, k_eq_v=0, v_norm=1), v=FAKE + 0x50) == UNSUPPORTED
    # the angle tables (8 bytes per position and pair: 16 positions of 128 rows with 8 q heads
    # per kv head) and q_norm_w share one 32 KiB key stage: 256 rotated dims fit, 512 do not
    assert _prefill_qp(_layer(W.GLOBAL_31B, rope_dims=512, rope_freq_dim=512)) == UNSUPPORTED
    assert "too large" in g.g4attn_last_error()
    assert _prefill_qp(_layer(W.GLOBAL_31B, rope_dims=256, rope_freq_dim=512), batch=0) == g.G4ATTN_OK
    assert _prefill_qp(G, batch=0) == g.G4ATTN_OK
