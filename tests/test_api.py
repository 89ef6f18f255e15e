"""C-ABI boundary checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before touching the HIP runtime.

No test here calls fa_fwd with arguments that pass validation (that would launch a kernel).
"""
import ctypes
import os
import re

import pytest

import exact_attention_58_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    fa.ensure_built()
    return fa.lib()


def header_functions():
    src = open(os.path.join(ROOT, "include", "fa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_\w+)\s*\(", src)))


def test_header_symbols_are_exported(L):
    names = header_functions()
    assert set(names) == {"fa_fwd", "fa_fwd_varlen", "fa_fwd_config", "fa_tune_fwd", "fa_tune_clear",
                          "fa_bwd", "fa_bwd_noalloc", "fa_status_str", "fa_select_config",
                          "fa_select_config_cus", "fa_version"}
    for n in names:
        assert hasattr(L, n), n
    assert set(fa.EXPORTED) == set(names)


def test_version_and_status_strings(L):
    assert L.fa_version() >= 1
    for code, word in [(0, "FA_OK"), (1, "FA_EINVAL"), (2, "FA_EUNSUPPORTED"), (3, "FA_ELAUNCH")]:
        assert fa.fa_status_str(code).startswith(word)
    assert "unknown" in fa.fa_status_str(99)


P = 4096  # a non-null, aligned fake pointer value: only ever passed with invalid arguments


def call(L, q=P, k=P, v=P, o=P, lse=P, B=1, H=1, Nq=8, Nk=8, d=64, scale=0.125, causal=0, dtype=2):
    return L.fa_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, ctypes.c_float(scale), causal, dtype, None)


@pytest.mark.parametrize("kw", [
    dict(q=None), dict(k=None), dict(v=None), dict(o=None), dict(lse=None),
    dict(B=0), dict(H=0), dict(Nq=0), dict(Nk=0), dict(d=0), dict(B=-1), dict(Nk=-5),
    dict(dtype=3), dict(dtype=-1),
    dict(scale=float("nan")), dict(scale=float("inf")), dict(scale=float("-inf")),
    dict(B=2**40, H=2**40),                   # B*H overflows
    dict(B=2**31, H=2**20, Nq=2**20, d=64),   # element count overflows int64
    dict(q=P + 1, dtype=2),                   # misaligned for a 2-byte element
    dict(o=P + 2, dtype=0),                   # misaligned for fp32
    dict(lse=P + 2),                          # misaligned fp32 lse
])
def test_invalid_arguments(L, kw):
    assert call(L, **kw) == fa.FA_EINVAL


@pytest.mark.parametrize("kw", [dict(d=257), dict(d=512), dict(d=129, dtype=0), dict(d=256, dtype=0),
                                dict(Nq=2**26, d=64), dict(Nk=2**25, d=128)])
def test_unsupported(L, kw):
    assert call(L, **kw) == fa.FA_EUNSUPPORTED


def call_varlen(L, q=P, k=P, v=P, o=P, lse=P, cq=P, ck=P, B=2, H=1, Tq=8, Tk=8, mq=4, mk=4, d=64,
                scale=0.125, causal=0, dtype=2):
    return L.fa_fwd_varlen(q, k, v, o, lse, cq, ck, B, H, Tq, Tk, mq, mk, d, ctypes.c_float(scale),
                           causal, dtype, None)


@pytest.mark.parametrize("kw", [
    dict(q=None), dict(o=None), dict(lse=None), dict(cq=None), dict(ck=None),
    dict(cq=P + 2), dict(ck=P + 1), dict(q=P + 1),
    dict(B=0), dict(H=0), dict(Tq=0), dict(Tk=0), dict(mq=0), dict(mk=0), dict(d=0),
    dict(mq=9), dict(mk=9), dict(dtype=5), dict(scale=float("nan")),
    dict(B=2**40, H=2**40),
])
def test_varlen_invalid_arguments(L, kw):
    assert call_varlen(L, **kw) == fa.FA_EINVAL


@pytest.mark.parametrize("kw", [dict(d=257), dict(d=129, dtype=0), dict(Tq=2**26, mq=2**26, d=64)])
def test_varlen_unsupported(L, kw):
    assert call_varlen(L, **kw) == fa.FA_EUNSUPPORTED


def call_cfg(L, cfg, q=P, B=1, H=1, Nq=8, Nk=8, d=64, causal=0, dtype=2, scale=0.125, occ=0, group=0):
    Br, Bc, waves = cfg
    return L.fa_fwd_config(q, P, P, P, P, B, H, Nq, Nk, d, ctypes.c_float(scale), causal, dtype,
                           Br, Bc, waves, occ, group, None)


@pytest.mark.parametrize("cfg,kw", [
    ((256, 64, 8), dict(dtype=0)),             # no fp32 ping-pong kernel
    ((128, 64, 4), dict(dtype=0, d=128)),      # fp32 d > 96 uses 32-key tiles
    ((128, 64, 4), dict(dtype=0)),             # fp32 up to d = 64: 128-key tiles on 16-byte rows
    ((128, 128, 4), dict(dtype=0, q=P + 4)),   # and 64-key tiles on rows off 16-byte alignment
    ((128, 128, 4), dict(dtype=0, d=96)),      # 128-key fp32 tiles only up to d = 64
    ((64, 128, 4), dict(dtype=0)),             # and not for the key split
    ((128, 32, 4), dict(dtype=2)),             # 16-bit tiles are 64 keys for 32 < d <= 224
    ((128, 64, 4), dict(dtype=2, d=32)),       # and 128 keys up to d = 32
    ((64, 64, 4), dict(dtype=1, d=20)),
    ((64, 32, 4), dict(dtype=0, d=128)),       # no fp32 key split above d = 96
    ((64, 64, 4), dict(d=136)),                # the 16-bit key split stops at d = 128
    ((256, 64, 8), dict(d=136)),               # ping-pong only up to d = 128
    ((256, 128, 8), dict(d=60)),               # and for d % 8 == 0
    ((256, 128, 8), dict(q=P + 2)),            # and for 16-byte aligned rows
    ((256, 64, 8), dict(d=64)),                # ping-pong tiles: 128 keys up to d = 64
    ((256, 128, 8), dict(d=96)),               # and 64 keys above
    ((512, 64, 16), dict()), ((128, 64, 8), dict()), ((0, 0, 0), dict()),
    ((128, 64, 4), dict(occ=5)), ((128, 64, 4), dict(occ=-1)),       # knob ranges
    ((128, 64, 4), dict(group=4)), ((128, 64, 4), dict(group=2048)),
    ((128, 64, 4), dict(group=-8)),
])
def test_fwd_config_unsupported(L, cfg, kw):
    """Configurations with no kernel are rejected before any HIP call."""
    assert call_cfg(L, cfg, **kw) == fa.FA_EUNSUPPORTED


def test_fwd_config_invalid_arguments(L):
    assert call_cfg(L, (128, 64, 4), B=0) == fa.FA_EINVAL
    assert call_cfg(L, (128, 64, 4), q=None) == fa.FA_EINVAL
    assert call_cfg(L, (128, 64, 4), scale=float("nan")) == fa.FA_EINVAL


def call_tune(L, reps=5, q=P, B=1, d=64, scale=0.125):
    out = [ctypes.c_int(-1) for _ in range(5)]
    rc = L.fa_tune_fwd(q, P, P, P, P, B, 1, 8, 8, d, ctypes.c_float(scale), 0, 2, reps, None,
                       *[ctypes.byref(x) for x in out])
    return rc, [x.value for x in out]


@pytest.mark.parametrize("kw", [dict(reps=0), dict(reps=1001), dict(q=None), dict(B=0), dict(d=0),
                                dict(scale=float("inf"))])
def test_tune_invalid_arguments(L, kw):
    rc, out = call_tune(L, **kw)
    assert rc == fa.FA_EINVAL and out == [-1] * 5


def test_tune_clear_needs_no_gpu(L):
    fa.fa_tune_clear()
    fa.fa_tune_clear()


def call_bwd(L, q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, delta=P, B=1, H=1, Nq=8, Nk=8, d=64,
             scale=0.125, causal=0, dtype=2):
    return L.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, delta, B, H, Nq, Nk, d, ctypes.c_float(scale),
                    causal, dtype, None)


@pytest.mark.parametrize("kw", [
    dict(q=None), dict(k=None), dict(v=None), dict(o=None), dict(lse=None), dict(do=None),
    dict(dq=None), dict(dk=None), dict(dv=None), dict(delta=None),
    dict(B=0), dict(Nq=0), dict(Nk=0), dict(d=0), dict(dtype=3),
    dict(scale=float("nan")), dict(B=2**40, H=2**40),
    dict(do=P + 1), dict(dv=P + 1), dict(lse=P + 2), dict(delta=P + 2),
    dict(q=P + 2, dtype=0), dict(dk=P + 2, dtype=0),   # fp32 buffers need 4-byte alignment
])
def test_bwd_invalid_arguments(L, kw):
    assert call_bwd(L, **kw) == fa.FA_EINVAL


@pytest.mark.parametrize("kw", [dict(d=136), dict(d=256), dict(d=129, dtype=0), dict(d=200, dtype=1)])
def test_bwd_unsupported(L, kw):
    """Head dims past 128 have no backward kernel (every dtype)."""
    assert call_bwd(L, **kw) == fa.FA_EUNSUPPORTED


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [129, 160, 200, 224, 256])
def test_select_config_large_head_dims(dtype, d):
    """Head dims past 128 (16-bit only): the 4-wave kernel compiled for the padded dim."""
    cfg = fa.fa_select_config(dtype, 4, 16, 4096, 4096, d, False)
    assert cfg["waves"] == 4 and cfg["Br"] == 128 and cfg["Bc"] == (32 if d > 224 else 64)
    assert cfg["dpad"] % 32 == 0 and d <= cfg["dpad"] < d + 32
    vpad = 64 if (cfg["dpad"] // 8) % 8 == 0 else 0
    lds = cfg["Bc"] * (cfg["dpad"] * 2 + 16) + cfg["Bc"] * (cfg["dpad"] * 2 + vpad)
    assert lds <= 160 * 1024


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [1, 5, 32, 33, 64, 96, 100, 128])
def test_select_config(dtype, d):
    cfg = fa.fa_select_config(dtype, 4, 16, 4096, 4096, d, False)
    assert cfg["dpad"] % 32 == 0 and d <= cfg["dpad"] < d + 32
    assert cfg["Br"] == 32 * cfg["waves"] or (cfg["waves"] == 4 and cfg["Br"] == 64)
    assert cfg["Bc"] in (32, 64, 128)
    s = 4 if dtype == "f32" else 2
    if cfg["waves"] == 8:
        # ping-pong kernel, one workgroup per CU
        assert dtype != "f32" and d % 8 == 0
        # three K and four V tile buffers; K rows padded to an odd chunk count, V rows to
        # 4 or 12 chunks mod 16
        kp = cfg["dpad"] // 8 + 1
        vp = cfg["dpad"] // 8 + (4 if cfg["dpad"] in (64, 128) else 0)
        lds = cfg["Bc"] * 16 * (3 * kp + 4 * vp)
        assert lds <= 160 * 1024
    else:
        # 4-wave kernel: K with a 16-byte row pad, V padded for its transposed reads
        vpad = 64 if (dtype != "f32" and cfg["dpad"] in (64, 128)) else 0
        lds = cfg["Bc"] * (cfg["dpad"] * s + 16) + cfg["Bc"] * (cfg["dpad"] * s + vpad)
        if cfg["Br"] == 64:
            lds *= 2  # key split: one tile buffer per key half
        assert lds * 2 <= 160 * 1024  # two workgroups per CU fit the 160 KiB LDS


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_select_config_grid_fill(dtype):
    """The 256-row kernel only when its grid gives every compute unit a workgroup."""
    big = fa.fa_select_config(dtype, 4, 16, 4096, 4096, 128, False, num_cus=256)
    assert big["waves"] == 8 and big["Br"] == 256 and big["Bc"] == 64
    big64 = fa.fa_select_config(dtype, 4, 16, 4096, 4096, 64, False, num_cus=256)
    assert big64["waves"] == 8 and big64["Bc"] == 128  # 128-key tiles up to d = 64
    small = fa.fa_select_config(dtype, 2, 12, 1000, 3001, 96, False, num_cus=256)
    # too few 128-row workgroups: 64 rows per workgroup, keys split between two waves
    assert small["waves"] == 4 and small["Br"] == 64
    small_causal = fa.fa_select_config(dtype, 2, 12, 1000, 3001, 96, True, num_cus=256)
    assert small_causal["waves"] == 4 and small_causal["Br"] == 64  # causal grids split too
    # between one and two 128-row workgroups per CU: causal grids split
    assert fa.fa_select_config(dtype, 1, 20, 2048, 2048, 64, True, num_cus=256)["Br"] == 64
    # non-causal: the ping-pong kernel down to 5/8 of a 256-row workgroup per CU; below it the
    # key split up to one 128-row workgroup per CU (1.5 for d <= 64), the 4-wave kernel above
    assert fa.fa_select_config(dtype, 1, 20, 2048, 2048, 64, False, num_cus=256)["Br"] == 256
    assert fa.fa_select_config(dtype, 1, 16, 2048, 2048, 64, False, num_cus=256)["Br"] == 64
    assert fa.fa_select_config(dtype, 1, 8, 4096, 4096, 96, False, num_cus=256)["Br"] == 64
    assert fa.fa_select_config(dtype, 1, 9, 4096, 4096, 96, False, num_cus=256)["Br"] == 128
    assert fa.fa_select_config(dtype, 1, 9, 4096, 4096, 64, False, num_cus=256)["Br"] == 64
    assert fa.fa_select_config(dtype, 1, 12, 4096, 4096, 32, False, num_cus=256)["Br"] == 64
    assert fa.fa_select_config(dtype, 1, 13, 4096, 4096, 32, False, num_cus=256)["Br"] == 128
    assert fa.fa_select_config(dtype, 1, 8, 4096, 4096, 128, False, num_cus=256)["Br"] == 64
    assert fa.fa_select_config(dtype, 1, 9, 4096, 4096, 128, False, num_cus=256)["Br"] == 128
    assert fa.fa_select_config(dtype, 1, 20, 2048, 2048, 64, True, num_cus=256)["waves"] == 4
    assert fa.fa_select_config(dtype, 1, 40, 2048, 2048, 64, True, num_cus=256)["Br"] == 128
    # causal grids of exactly two 128-row workgroups per CU: the key split up to d = 96, the
    # ping-pong kernel at d = 128; three per CU: the ping-pong kernel
    assert fa.fa_select_config(dtype, 1, 16, 4096, 4096, 64, True, num_cus=256)["Br"] == 64
    assert fa.fa_select_config(dtype, 1, 8, 8192, 8192, 64, True, num_cus=256)["Br"] == 64
    assert fa.fa_select_config(dtype, 2, 8, 4096, 4096, 96, True, num_cus=256)["Br"] == 64
    assert fa.fa_select_config(dtype, 1, 16, 4096, 4096, 128, True, num_cus=256)["waves"] == 8
    assert fa.fa_select_config(dtype, 1, 32, 3072, 3072, 64, True, num_cus=256)["waves"] == 8
    small_d128 = fa.fa_select_config(dtype, 2, 12, 1000, 3001, 128, False, num_cus=256)
    assert small_d128["Br"] == 64  # the key split reaches d = 128 for 16-bit inputs
    # enough 128-row workgroups (d % 8 != 0 keeps the 256-row kernel out): no key split
    filled = fa.fa_select_config(dtype, 4, 16, 1000, 3001, 90, False, num_cus=256)
    assert filled["Br"] == 128
    odd_d = fa.fa_select_config(dtype, 4, 16, 4096, 4096, 100, False, num_cus=256)
    assert odd_d["waves"] == 4
    # short key sequences (HBM-bound) stay on the 4-wave kernel
    short = fa.fa_select_config(dtype, 64, 128, 128, 128, 128, False, num_cus=256)
    assert short["waves"] == 4
    edge = fa.fa_select_config(dtype, 16, 128, 512, 512, 128, False, num_cus=256)
    assert edge["waves"] == 4
    longer = fa.fa_select_config(dtype, 8, 128, 1024, 513, 128, False, num_cus=256)
    assert longer["waves"] == 8
    # non-causal d <= 96 with three or more 128-row workgroups per CU: the 4-wave kernel up
    # to 1536 keys; fewer per CU, more keys or d = 128: the ping-pong kernel
    assert fa.fa_select_config(dtype, 4, 16, 1536, 1536, 64, False, num_cus=256)["waves"] == 4
    assert fa.fa_select_config(dtype, 16, 16, 1024, 1024, 48, False, num_cus=256)["waves"] == 4
    assert fa.fa_select_config(dtype, 2, 16, 1536, 1536, 64, False, num_cus=256)["waves"] == 8
    assert fa.fa_select_config(dtype, 4, 16, 2048, 1537, 64, False, num_cus=256)["waves"] == 8
    assert fa.fa_select_config(dtype, 16, 16, 1024, 1024, 96, False, num_cus=256)["waves"] == 4
    assert fa.fa_select_config(dtype, 16, 16, 1024, 1024, 128, False, num_cus=256)["waves"] == 8
    assert fa.fa_select_config(dtype, 16, 16, 1024, 1024, 64, True, num_cus=256)["waves"] == 4
    # head dims up to 32: the 4-wave kernel at every length
    for causal in (False, True):
        assert fa.fa_select_config(dtype, 4, 16, 16384, 16384, 32, causal, num_cus=256)["waves"] == 4
    # causal grids keep the 4-wave kernel up to 2048 keys (d > 64) or 2560 keys (d <= 64;
    # 4096 on grids of eight or more 128-row workgroups per CU)
    for B, d, last_4wave in ((4, 128, 2048), (4, 96, 2048), (2, 64, 2560), (4, 64, 4096)):
        at = fa.fa_select_config(dtype, B, 32, last_4wave, last_4wave, d, True, num_cus=256)
        past = fa.fa_select_config(dtype, B, 32, last_4wave + 1, last_4wave + 1, d, True, num_cus=256)
        assert at["waves"] == 4 and past["waves"] == 8, (d, at, past)
        assert fa.fa_select_config(dtype, B, 32, last_4wave, last_4wave, d, False, num_cus=256)["waves"] == 8


def test_select_config_fp32_key_split():
    """fp32 grids too small to fill the chip take the two-way key split (causal too), and
    the smallest the four-way split."""
    small = fa.fa_select_config("f32", 1, 16, 1024, 1024, 64, False, num_cus=256)
    assert (small["Br"], small["Bc"], small["waves"]) == (64, 64, 4)
    small128 = fa.fa_select_config("f32", 1, 8, 1024, 1024, 128, False, num_cus=256)
    assert (small128["Br"], small128["Bc"]) == (128, 32)  # no split above d = 96
    assert fa.fa_select_config("f32", 4, 4, 4096, 4096, 64, False, num_cus=256)["Br"] == 128
    # four-way split: at most one 32-row workgroup per CU (causal grids: four, two for d = 96)
    tiny = fa.fa_select_config("f32", 1, 1, 256, 256, 64, True, num_cus=256)
    assert (tiny["Br"], tiny["Bc"], tiny["waves"]) == (32, 32, 4)
    assert fa.fa_select_config("f32", 1, 8, 1024, 1024, 64, False, num_cus=256)["Br"] == 32
    assert fa.fa_select_config("f32", 1, 8, 1024, 1024, 64, True, num_cus=256)["Br"] == 32
    assert fa.fa_select_config("f32", 1, 2, 4096, 4096, 64, False, num_cus=256)["Br"] == 32
    assert fa.fa_select_config("f32", 1, 4, 4096, 4096, 64, False, num_cus=256)["Br"] == 64
    assert fa.fa_select_config("f32", 1, 16, 2048, 2048, 64, True, num_cus=256)["Br"] == 32
    assert fa.fa_select_config("f32", 1, 16, 2048, 2048, 32, False, num_cus=256)["Br"] == 64
    assert fa.fa_select_config("f32", 2, 4, 512, 512, 96, True, num_cus=256)["Br"] == 32
    assert fa.fa_select_config("f32", 2, 16, 512, 512, 96, True, num_cus=256)["Br"] == 32
    assert fa.fa_select_config("f32", 1, 16, 2048, 2048, 96, True, num_cus=256)["Br"] == 64
    assert fa.fa_select_config("f32", 2, 4, 1024, 1024, 96, False, num_cus=256)["Br"] == 32
    assert fa.fa_select_config("f32", 1, 8, 2048, 2048, 64, True, num_cus=64)["Br"] == 64
    assert fa.fa_select_config("f32", 1, 1, 256, 128, 64, True, num_cus=256)["Br"] == 128  # too few keys
    # up to two 128-row workgroups per CU (fp32, causal or not)
    assert fa.fa_select_config("f32", 1, 20, 2048, 2048, 64, False, num_cus=256)["Br"] == 64
    assert fa.fa_select_config("f32", 1, 40, 2048, 2048, 64, False, num_cus=256)["Br"] == 128
    # causal fp32 splits up to four per CU
    assert fa.fa_select_config("f32", 1, 16, 4096, 4096, 64, True, num_cus=256)["Br"] == 64
    assert fa.fa_select_config("f32", 1, 64, 4096, 4096, 64, True, num_cus=256)["Br"] == 128
    assert fa.fa_select_config("f32", 1, 8, 1024, 128, 64, False, num_cus=256)["Br"] == 128
    # non-causal d = 96 splits only below one per CU (the split runs one wave per SIMD there)
    assert fa.fa_select_config("f32", 1, 8, 2048, 2048, 96, False, num_cus=256)["Br"] == 64
    assert fa.fa_select_config("f32", 2, 16, 1024, 1024, 96, False, num_cus=256)["Br"] == 128
    assert fa.fa_select_config("f32", 2, 16, 1024, 1024, 96, True, num_cus=256)["Br"] == 64


def test_select_config_errors():
    with pytest.raises(fa.FaError) as e:
        fa.fa_select_config("bf16", 1, 1, 16, 16, 257, False)
    assert e.value.status == fa.FA_EUNSUPPORTED
    with pytest.raises(fa.FaError) as e:
        fa.fa_select_config("f32", 1, 1, 16, 16, 129, False)
    assert e.value.status == fa.FA_EUNSUPPORTED
    with pytest.raises(fa.FaError) as e:
        fa.fa_select_config("bf16", 0, 1, 16, 16, 64, False)
    assert e.value.status == fa.FA_EINVAL


def test_product_never_touches_oracle():
    """The product package never imports the oracle, and the native sources never name it."""
    pkg = os.path.join(ROOT, "exact_attention_58_amd")
    imp = re.compile(r"^\s*(import\s+oracle|from\s+oracle|from\s+\.\.?\s*oracle)", re.M)
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            text = open(os.path.join(dirpath, f), errors="ignore").read() if f.endswith(
                (".py", ".hip", ".cpp", ".h")) else ""
            if f.endswith(".py"):
                assert not imp.search(text), f
                assert "attn_oracle" not in text and "importlib" not in text, f
            elif text:
                assert "oracle" not in text.lower(), f
    assert "oracle" not in open(os.path.join(ROOT, "include", "fa.h")).read().lower()


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(fa, "LIB_PATH", str(tmp_path / "nope.so"))
    monkeypatch.setattr(fa, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        fa.lib()


def test_select_config_current_device_matches_pure_rule(L):
    """The section-8(b) signature reads the current device's CU count; without a visible device
    it takes MI355X's 256, the same answer as the pure variant given 256."""
    import torch
    if torch.cuda.is_available():
        cus = torch.cuda.get_device_properties(0).multi_processor_count
    else:
        cus = 256
    for args in (("bf16", 4, 16, 4096, 4096, 128, False), ("f16", 2, 12, 1000, 3001, 96, False),
                 ("f32", 1, 1, 256, 256, 64, True), ("bf16", 1, 8, 16384, 16384, 64, True)):
        dev = fa.fa_select_config(*args, num_cus=None)
        pure = fa.fa_select_config(*args, num_cus=cus)
        assert dev == {k: pure[k] for k in ("Br", "Bc", "waves")}, args
    with pytest.raises(fa.FaError) as e:
        fa.fa_select_config("bf16", 1, 1, 16, 16, 257, False, num_cus=None)
    assert e.value.status == fa.FA_EUNSUPPORTED
