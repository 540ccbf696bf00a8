"""The C ABI without a GPU: the library loads, exports every function that
include/pa.h declares, and rejects bad host arguments before any launch."""

import ctypes
import os
import re

import pytest

from paged_kv_cache_234_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "pa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(pa_[a-z_0-9]+)\s*\(", text,
                                 flags=re.M)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(_lib.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for s in range(5):
        assert _lib.status_string(s).startswith("PA_")
    assert _lib.status_string(99) == "PA_ERR_UNKNOWN"


def test_workspace_bytes():
    assert _lib.pa_decode_workspace_bytes(8, 32, 128, 256) == 8 * 32 * 256 * 4 * 130
    assert _lib.pa_decode_workspace_bytes(-1, 32, 128, 256) == 0


def _decode(lib, **kw):
    a = dict(out=None, q=None, q_dt=1, k=None, v=None, c_dt=1, ks=None, vs=None, bt=None, W=4,
             lens=None, B=2, hq=8, hkv=2, d=128, bs=16, scale=0.1, ps=0, pmax=1)
    a.update(kw)
    return lib.pa_decode(a["out"], a["q"], a["q_dt"], a["k"], a["v"], a["c_dt"], a["ks"], a["vs"],
                         a["bt"], a["W"], a["lens"], a["B"], a["hq"], a["hkv"], a["d"], a["bs"],
                         a["scale"], a["ps"], a["pmax"], None, None, None, None)


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


@pytest.mark.parametrize("kw,status", [
    (dict(), _lib.PA_ERR_ARG),                                    # null pointers
    (dict(hq=7, hkv=2), _lib.PA_ERR_ARG),                         # Hq not a multiple of Hkv
    (dict(d=96), _lib.PA_ERR_UNSUPPORTED),
    (dict(bs=32), _lib.PA_ERR_UNSUPPORTED),
    (dict(hq=34, hkv=2), _lib.PA_ERR_UNSUPPORTED),                # G = 17
    (dict(q_dt=0, c_dt=1), _lib.PA_ERR_UNSUPPORTED),              # f32 q over bf16 cache
    (dict(q_dt=1, c_dt=2), _lib.PA_ERR_ARG),                      # fp8 without scales
    (dict(q_dt=5), _lib.PA_ERR_ARG),
    (dict(B=-1), _lib.PA_ERR_ARG),
    (dict(B=0), _lib.PA_OK),                                      # empty batch: nothing to do
])
def test_decode_argument_validation(kw, status):
    lib = _lib.load()
    assert _decode(lib, **kw) == status


def test_decode_rejects_bad_partitioning():
    lib = _lib.load()
    common = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, lens=FAKE)
    assert _decode(lib, ps=24, pmax=4, **common) == _lib.PA_ERR_ARG       # not a multiple of 16
    assert _decode(lib, ps=32, pmax=4, **common) == _lib.PA_ERR_ARG       # no partial buffers
    assert _decode(lib, ps=-16, **common) == _lib.PA_ERR_ARG
    assert _decode(lib, scale=float("nan"), **common) == _lib.PA_ERR_ARG


def test_append_reduce_prefill_validation():
    lib = _lib.load()
    # append: fp8 cache needs scales; zero tokens is a no-op
    assert lib.pa_kv_append(FAKE, FAKE, 1, FAKE, FAKE, 2, None, None, FAKE, 4, 8, 2, 128, 16,
                            None) == _lib.PA_ERR_ARG
    assert lib.pa_kv_append(None, None, 1, None, None, 1, None, None, None, 0, 8, 2, 128, 16,
                            None) == _lib.PA_OK
    assert lib.pa_kv_append(FAKE, FAKE, 0, FAKE, FAKE, 2, FAKE, FAKE, FAKE, 4, 8, 2, 128, 16,
                            None) == _lib.PA_ERR_UNSUPPORTED
    # reduce: too many partitions for the LDS weight table
    assert lib.pa_decode_splitk_reduce(FAKE, 1, FAKE, FAKE, FAKE, FAKE, 2, 8, 128, 512, 5000,
                                       None) == _lib.PA_ERR_UNSUPPORTED
    assert lib.pa_decode_splitk_reduce(FAKE, 1, FAKE, FAKE, FAKE, FAKE, 2, 8, 128, 0, 4,
                                       None) == _lib.PA_ERR_ARG
    # prefill: nothing to do for zero chunks; null pointers rejected otherwise
    assert lib.pa_prefill_chunk(None, None, 1, None, 0, 0, None, None, 1, None, None, None, 4,
                                None, 8, 2, 128, 16, 0.1, None) == _lib.PA_OK
    assert lib.pa_prefill_chunk(None, None, 1, None, 2, 64, None, None, 1, None, None, None, 4,
                                None, 8, 2, 128, 16, 0.1, None) == _lib.PA_ERR_ARG


def test_cascade_validation():
    lib = _lib.load()

    def call(ps=256, pmax=4, B=4, ng=1, mgs=4, gs=FAKE, gq=FAKE, gp=FAKE, parts=FAKE, plan=None,
             nbytes=0):
        return lib.pa_decode_cascade(FAKE, 1, None, None, None, FAKE, FAKE, 1, None, None, FAKE, 32,
                                     FAKE, B, gs,
                                     gq, gp, ng, mgs, 8, 2, 128, 16, 0.1, ps, pmax, parts, parts,
                                     parts, plan, nbytes, None)

    assert call(ps=0) == _lib.PA_ERR_ARG                         # split-K only
    assert call(parts=None) == _lib.PA_ERR_ARG                   # partial buffers required
    assert call(gs=None) == _lib.PA_ERR_ARG                      # group arrays required
    assert call(ng=-1) == _lib.PA_ERR_ARG
    assert call(mgs=-1) == _lib.PA_ERR_ARG
    assert call(B=4000, ng=200) == _lib.PA_ERR_UNSUPPORTED       # more than 4096 rows
    assert call(plan=FAKE, nbytes=64) == _lib.PA_ERR_ARG          # plan buffer too small
    assert call(B=0) == _lib.PA_OK


def test_multi_query_validation():
    lib = _lib.load()

    def call(ps=64, pmax=4, B=4, mq=8, qsl=FAKE, parts=FAKE, plan=None, nbytes=0,
             new=(None, None, None)):
        return lib.pa_decode_multi(FAKE, 1, *new, qsl, mq, FAKE, FAKE, 1, None, None, FAKE, 32,
                                   FAKE, B, 8, 2, 128, 16, 0.1, ps, pmax, parts, parts, parts,
                                   plan, nbytes, None)

    assert call(ps=0) == _lib.PA_ERR_ARG
    assert call(new=(FAKE, None, FAKE)) == _lib.PA_ERR_ARG       # append arrays: all or none
    assert call(new=(None, None, FAKE)) == _lib.PA_ERR_ARG
    assert call(parts=None) == _lib.PA_ERR_ARG
    assert call(qsl=None) == _lib.PA_ERR_ARG
    assert call(mq=-1) == _lib.PA_ERR_ARG
    assert call(mq=65) == _lib.PA_ERR_UNSUPPORTED
    assert call(mq=0) == _lib.PA_OK
    assert call(B=0) == _lib.PA_OK


def test_decode_append_validation():
    lib = _lib.load()

    def call(out=FAKE, kn=FAKE, vn=FAKE, sl=FAKE, ps=64, parts=FAKE, B=4, plan=None, nbytes=0):
        return lib.pa_decode_append(out, FAKE, 1, kn, vn, sl, FAKE, FAKE, 1, None, None, FAKE, 32,
                                    FAKE, B, 8, 2, 128, 16, 0.1, ps, 4, parts, parts, parts, plan,
                                    nbytes, None)

    assert call(vn=None) == _lib.PA_ERR_ARG                       # append arrays go together
    assert call(sl=None) == _lib.PA_ERR_ARG
    assert call(parts=None) == _lib.PA_ERR_ARG
    assert call(ps=0, out=None) == _lib.PA_ERR_ARG
    assert call(plan=FAKE, nbytes=64) == _lib.PA_ERR_ARG              # plan buffer too small
    assert call(B=0) == _lib.PA_OK


def test_decode_plan_validation():
    lib = _lib.load()

    def call(plan=FAKE, nbytes=1 << 20, entry=0, B=4, hq=8, hkv=2, d=128, c_dt=1, ps=64, pmax=4,
             gs=None, ng=0, qsl=None, mq=0):
        return lib.pa_decode_plan(plan, nbytes, entry, FAKE, 32, FAKE, B, None, gs, gs, gs, ng, 4,
                                  qsl, mq, hq, hkv, d, c_dt, ps, pmax, None)

    assert call(plan=None) == _lib.PA_ERR_ARG
    assert call(entry=3) == _lib.PA_ERR_ARG
    assert call(entry=1, ng=2) == _lib.PA_ERR_ARG                 # groups without their arrays
    assert call(entry=1, ps=0) == _lib.PA_ERR_ARG                 # cascade plans are split-K
    assert call(entry=2, mq=8) == _lib.PA_ERR_ARG                 # no query map
    assert call(entry=2, mq=65, qsl=FAKE) == _lib.PA_ERR_UNSUPPORTED
    assert call(entry=1, B=4000, ng=200, gs=FAKE) == _lib.PA_ERR_UNSUPPORTED
    assert call(nbytes=64) == _lib.PA_ERR_ARG                     # smaller than the plan
    assert call(hq=7) == _lib.PA_ERR_ARG
    assert call(d=96) == _lib.PA_ERR_UNSUPPORTED
    assert call(ps=24) == _lib.PA_ERR_ARG
    assert call(B=5000) == _lib.PA_ERR_UNSUPPORTED
    assert call(B=0, plan=None) == _lib.PA_OK
    # header + three row arrays (16-aligned) + 16 words per wavefront of the
    # largest grid (one workgroup of 4 per CU and wave slot)
    assert lib.pa_decode_plan_bytes(64, 1, 128) % 64 == 0
    assert lib.pa_decode_plan_bytes(64, 1, 64) > lib.pa_decode_plan_bytes(64, 1, 128)
    assert lib.pa_decode_plan_bytes(-1, 1, 128) == 0
    assert lib.pa_decode_plan_bytes(64, 1, 96) == 0


def _noalloc(lib, **kw):
    a = dict(out=FAKE, q=FAKE, q_dt=1, k=FAKE, v=FAKE, c_dt=1, ks=None, vs=None, bt=FAKE, W=4,
             lens=FAKE, B=2, hq=8, hkv=2, d=128, bs=16, scale=0.1, ps=64, pmax=4)
    a.update(kw)
    return lib.pa_decode_noalloc(a["out"], a["q"], a["q_dt"], a["k"], a["v"], a["c_dt"], a["ks"],
                                 a["vs"], a["bt"], a["W"], a["lens"], a["B"], a["hq"], a["hkv"],
                                 a["d"], a["bs"], a["scale"], a["ps"], a["pmax"], None)


def test_noalloc_rejects_bad_arguments_and_oversized_partials_before_any_device_call():
    """Every host check runs before the device is touched: partials beyond
    the static scratch (64 MiB) are PA_ERR_TOO_LARGE, split-K is required."""
    lib = _lib.load()
    assert lib.pa_decode_noalloc_max_bytes() == 64 << 20
    assert _noalloc(lib, ps=0) == _lib.PA_ERR_ARG
    assert _noalloc(lib, ps=24) == _lib.PA_ERR_ARG
    assert _noalloc(lib, pmax=0) == _lib.PA_ERR_ARG
    assert _noalloc(lib, out=None) == _lib.PA_ERR_ARG
    assert _noalloc(lib, d=96) == _lib.PA_ERR_UNSUPPORTED
    assert _noalloc(lib, B=0) == _lib.PA_OK
    # 8 x 32 heads x 512 partitions x 130 floats = 65 MiB of partials > 64 MiB
    assert _noalloc(lib, B=8, hq=32, hkv=8, pmax=512) == _lib.PA_ERR_TOO_LARGE
    assert _noalloc(lib, B=4096, hq=16, pmax=64) == _lib.PA_ERR_TOO_LARGE


def test_read_probe_rejects_bad_arguments_before_any_launch():
    lib = _lib.load()
    probe = lambda buf, nbytes, ids, n, sink, sink_bytes: lib.pa_read_probe(
        buf, nbytes, ids, n, sink, sink_bytes, None)
    assert probe(None, 1 << 20, FAKE, 4, FAKE, 1 << 20) == _lib.PA_ERR_ARG
    assert probe(FAKE, 1 << 20, FAKE, 0, FAKE, 1 << 20) == _lib.PA_ERR_ARG
    assert probe(FAKE, 2048, FAKE, 1, FAKE, 1 << 20) == _lib.PA_ERR_ARG          # < one chunk
    assert probe(FAKE, 1 << 20, FAKE, 257, FAKE, 1 << 20) == _lib.PA_ERR_ARG     # > 256 chunks
    assert probe(FAKE, 1 << 20, FAKE, 4, FAKE, 64) == _lib.PA_ERR_ARG            # sink too small
