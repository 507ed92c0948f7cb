"""C-ABI boundary checks that need no GPU: the library loads, exports every
function include/mla_decode.h declares, and rejects bad arguments on the
host before touching a device."""
import ctypes
import os
import re

import pytest

import mla_paged_kv_metadata_amd as mla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_decode.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_calls():
    names = _declared()
    for n in ("mla_get_metadata", "mla_decode_fwd", "mla_num_parts", "mla_workspace_bytes", "mla_status_str",
              "mla_get_metadata_ex"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = mla.load_library()
    for n in _declared():
        assert hasattr(lib, n), n


def test_status_strings():
    lib = mla.load_library()
    for s in range(6):
        assert lib.mla_status_str(s)
    assert lib.mla_status_str(0) == b"ok"


def test_workspace_bytes():
    n = mla.mla_workspace_bytes(64, 1, 128, 1, 512, 256)
    slots = 64 + 256
    assert n >= slots * 128 * 512 * 2 + slots * 128 * 4      # bf16 partial outputs, fp32 lse
    # Partial outputs are kept in whole 32-row blocks per KV head: 20 rows take a block
    # of 32, and 48 rows (s_q 3 x 16 heads) two blocks, for each of 2 KV heads.
    n = mla.mla_workspace_bytes(2, 1, 20, 1, 512, 8)
    assert n >= (2 + 8) * 32 * 512 * 2 + (2 + 8) * 20 * 4
    n = mla.mla_workspace_bytes(3, 3, 32, 2, 512, 5)
    assert n >= (3 + 5) * 2 * 64 * 512 * 2 + (3 + 5) * 2 * 48 * 4
    with pytest.raises(mla.MlaError) as e:
        mla.mla_workspace_bytes(0, 1, 128, 1, 512, 256)
    assert e.value.status == 1
    with pytest.raises(mla.MlaError):
        mla.mla_workspace_bytes(2, 1, 6, 4, 512, 8)      # heads not divisible


def _decode(lib, **kw):
    a = dict(q=1, batch=2, s_q=1, hq=16, d=576, kv=1, dt=0, nb=8, page=64, hk=1, bt=1, maxb=5, sl=1, dv=512,
             scale=1 / 24, vs=1.0, causal=0, md=1, parts=4, ns=1, ws=1, wsb=1 << 30, out=1, lse=1, stream=0)
    a.update(kw)
    P = ctypes.c_void_p
    return lib.mla_decode_fwd(P(a["q"]), a["batch"], a["s_q"], a["hq"], a["d"], P(a["kv"]), a["dt"], a["nb"],
                              a["page"], a["hk"], P(a["bt"]), a["maxb"], P(a["sl"]), a["dv"], a["scale"],
                              a["vs"], a["causal"], P(a["md"]), a["parts"], P(a["ns"]), P(a["ws"]), a["wsb"],
                              P(a["out"]), P(a["lse"]), P(a["stream"]))


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), 1), (dict(out=0), 1), (dict(lse=0), 1), (dict(batch=0), 1), (dict(hq=6, hk=4), 1),
    (dict(causal=2), 1), (dict(scale=float("nan")), 1), (dict(scale=-0.5), 2), (dict(d=192), 2), (dict(dv=128), 2),
    (dict(page=24), 2), (dict(page=8), 2), (dict(page=0), 1), (dict(dt=7), 2), (dict(s_q=9, hq=128), 2), (dict(batch=9000), 2),
    (dict(wsb=16), 3), (dict(ws=0), 3),
])
def test_decode_rejects_bad_arguments_before_any_device_call(kw, status):
    # Pointers are dummies: a rejected call must never dereference or launch.
    assert _decode(mla.load_library(), **kw) == status


def test_metadata_rejects_bad_arguments():
    lib = mla.load_library()
    P = ctypes.c_void_p
    assert lib.mla_get_metadata_ex(P(1), 0, 128, 1, 4, 2, P(1), P(1), P(0)) == 1
    assert lib.mla_get_metadata_ex(P(1), 4, 128, 1, 0, 2, P(1), P(1), P(0)) == 1
    assert lib.mla_get_metadata_ex(P(1), 4, 128, 1, 4, 0, P(1), P(1), P(0)) == 1
    assert lib.mla_get_metadata_ex(P(0), 4, 128, 1, 4, 2, P(1), P(1), P(0)) == 1
    assert lib.mla_get_metadata_ex(P(1), 9000, 128, 1, 4, 2, P(1), P(1), P(0)) == 2
    assert lib.mla_num_parts(4, 128, 1, None) == 1


def test_python_wrapper_rejects_cpu_tensors():
    import torch
    with pytest.raises((ValueError, TypeError)):
        mla.mla_get_metadata(torch.zeros(4, dtype=torch.int32), 128, 1)


def test_no_device_is_reported_when_arguments_are_valid():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    lib = mla.load_library()
    assert _decode(lib) == 4
    n = ctypes.c_int(0)
    assert lib.mla_num_parts(4, 128, 1, ctypes.byref(n)) == 4


def _decode_ext(lib, ext, **kw):
    a = dict(q=1, batch=2, s_q=1, hq=16, d=576, kv=1, dt=0, nb=8, page=64, hk=1, bt=1, maxb=5, sl=1, dv=512,
             scale=1 / 24, vs=1.0, causal=0, md=1, parts=4, ns=1, ws=1, wsb=1 << 30, out=1, lse=1, stream=0)
    a.update(kw)
    P = ctypes.c_void_p
    return lib.mla_decode_fwd_ext(P(a["q"]), a["batch"], a["s_q"], a["hq"], a["d"], P(a["kv"]), a["dt"], a["nb"],
                                  a["page"], a["hk"], P(a["bt"]), a["maxb"], P(a["sl"]), a["dv"], a["scale"],
                                  a["vs"], a["causal"], P(a["md"]), a["parts"], P(a["ns"]), P(a["ws"]), a["wsb"],
                                  P(a["out"]), P(a["lse"]), P(a["stream"]),
                                  None if ext is None else ctypes.byref(ext))


def test_header_declares_the_ext_struct_with_the_binding_layout():
    src = open(HEADER).read()
    body = re.search(r"typedef struct mla_decode_ext \{(.*?)\} mla_decode_ext;", src, flags=re.S).group(1)
    fields = re.findall(r"\b(\w+);", body)
    assert fields == [f for f, _ in mla.DecodeExt._fields_]


@pytest.mark.parametrize("stages,status", [(-1, 1), (4, 1)])
def test_ext_rejects_bad_stages_before_any_device_call(stages, status):
    ext = mla.DecodeExt(None, None, None, None, None, stages)
    assert _decode_ext(mla.load_library(), ext) == status


def test_ext_applies_the_plain_checks():
    lib = mla.load_library()
    ext = mla.DecodeExt(None, None, None, None, None, 0)
    assert _decode_ext(lib, ext, q=0) == 1
    assert _decode_ext(lib, None, scale=-1.0) == 2
    assert _decode_ext(lib, ext, wsb=16) == 3


@pytest.mark.parametrize("q_dtype,dt,q_rope,status", [
    (2, 1, None, 2),        # unknown q dtype
    (-1, 0, None, 2),
    (1, 0, None, 2),        # fp8 q with a bf16 cache
    (1, 1, 1, 2),           # fp8 q with a split query
])
def test_ext_rejects_unsupported_query_forms_before_any_device_call(q_dtype, dt, q_rope, status):
    ext = mla.DecodeExt(None, None, None, None, q_rope, 0, None, None, None, q_dtype)
    assert _decode_ext(mla.load_library(), ext, dt=dt) == status


def test_python_wrapper_checks_descale_and_fp8_query_forms():
    import torch
    q = torch.zeros((1, 1, 16, 576), dtype=torch.bfloat16)
    kv = torch.zeros((2, 64, 1, 576), dtype=torch.float8_e4m3fn)
    bt = torch.zeros((1, 2), dtype=torch.int32)
    sl = torch.zeros((1,), dtype=torch.int32)
    md = torch.zeros((4, 8), dtype=torch.int32)
    ns = torch.zeros((2,), dtype=torch.int32)
    with pytest.raises(ValueError):      # one factor per query head
        mla.mla_decode_fwd(q, kv, bt, sl, 512, md, ns, qk_descale=torch.ones(8))
    with pytest.raises(TypeError):       # fp32 factors
        mla.mla_decode_fwd(q, kv, bt, sl, 512, md, ns, pv_descale=torch.ones(16, dtype=torch.float64))
    with pytest.raises(ValueError):      # one base-2 scale
        mla.mla_decode_fwd(q, kv, bt, sl, 512, md, ns, bmm1_scale_log2_tensor=torch.ones(2))
    q8 = torch.zeros((1, 1, 16, 512), dtype=torch.float8_e4m3fn)
    with pytest.raises(ValueError):      # an fp8 query is joined
        mla.mla_decode_fwd(q8, kv[..., :512].contiguous(), bt, sl, 512, md, ns,
                           q_rope=torch.zeros((1, 1, 16, 64), dtype=torch.bfloat16))


def test_python_wrapper_checks_split_layout_shapes():
    import torch
    q = torch.zeros((1, 1, 16, 576), dtype=torch.bfloat16)
    kv = torch.zeros((2, 64, 1, 512), dtype=torch.bfloat16)
    bt = torch.zeros((1, 2), dtype=torch.int32)
    sl = torch.zeros((1,), dtype=torch.int32)
    md = torch.zeros((4, 8), dtype=torch.int32)
    ns = torch.zeros((2,), dtype=torch.int32)
    with pytest.raises(ValueError):      # kv_rope of the wrong width
        mla.mla_decode_fwd(q, kv, bt, sl, 512, md, ns, kv_rope=torch.zeros((2, 64, 1, 32), dtype=torch.bfloat16))
    with pytest.raises(ValueError):      # q_rope with a 576-wide q
        mla.mla_decode_fwd(q, kv, bt, sl, 512, md, ns, q_rope=torch.zeros((1, 1, 16, 64), dtype=torch.bfloat16))


def test_noalloc_refuses_oversized_problems_before_any_device_call():
    # mla_workspace_bytes for 4096 sequences x 1024 rows is far above the
    # static scratch; the call must fail before touching a device (dummy pointers).
    lib = mla.load_library()
    P = ctypes.c_void_p
    rc = lib.mla_decode_fwd_noalloc(P(1), 4096, 8, 128, 576, P(1), 0, 8, 64, 1, P(1), 1, P(1), 512, 0.04, 1.0, 0,
                                    P(1), 256, P(1), P(1), P(1), P(0))
    assert rc == 3
    assert b"scratch" in lib.mla_status_str(rc)
    n = mla.mla_workspace_bytes(4096, 8, 128, 1, 512, 256)
    assert n > mla.NOALLOC_SCRATCH_BYTES
    # Invalid sizes are INVALID_ARG, as for mla_decode_fwd.
    assert lib.mla_decode_fwd_noalloc(P(1), 0, 1, 16, 576, P(1), 0, 8, 64, 1, P(1), 1, P(1), 512, 0.04, 1.0, 0,
                                      P(1), 4, P(1), P(1), P(1), P(0)) == 1


def test_lds_dma_read_rejects_bad_sizes_before_any_device_call():
    lib = mla.load_library()
    P = ctypes.c_void_p
    assert lib.mla_lds_dma_read(P(0), 1024, P(0)) == 1
    assert lib.mla_lds_dma_read(P(1), 0, P(0)) == 1
    assert lib.mla_lds_dma_read(P(1), 1000, P(0)) == 1
