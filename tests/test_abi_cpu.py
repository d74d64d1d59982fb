"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re
import subprocess

import pytest

import sparse_mixture_experts_02_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(moe_\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moe.LIB_PATH):
        pytest.fail("libmoe.so is not built (run python -m sparse_mixture_experts_02_amd.build)")
    return moe.load_library()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("moe_forward", "moe_forward_timed", "moe_forward_routed", "moe_dispatch", "moe_dispatch_routed",
              "moe_workspace_bytes", "moe_status_string", "moe_abi_version"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for n in declared_functions():
        assert n in exported, n
        assert getattr(lib, n) is not None


def test_desc_layout_matches_header():
    # int64 T, D, F then seven int32 fields
    assert ctypes.sizeof(moe.MoeDesc) == 3 * 8 + 7 * 4 + 4  # padded to 8
    assert moe.MoeDesc.E.offset == 24 and moe.MoeDesc.deterministic.offset == 48


def test_routing_layout_matches_header():
    # two pointers, float (padded), double, int64, two pointers
    R = moe.MoeRouting
    assert ctypes.sizeof(R) == 56
    assert (R.replay_experts.offset, R.replay_mask.offset, R.dynamic_threshold.offset, R.capacity_factor.offset,
            R.seq_len.offset, R.kept.offset, R.stats.offset) == (0, 8, 16, 24, 32, 40, 48)
    assert moe.stats_len(8) == 28


def test_abi_version_and_strings(lib):
    assert moe.moe_abi_version() == 2
    for code in range(6):
        assert len(moe.moe_status_string(code)) > 0
    assert moe.moe_status_string(99) == "unknown status"


def _desc(**kw):
    base = dict(T=16, D=64, F=128, E=8, K=2, norm_topk=1, act=0, dtype=0, out_dtype=0, deterministic=0)
    base.update(kw)
    return moe.MoeDesc(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(K=0), moe.MOE_EINVAL), (dict(K=9), moe.MOE_EINVAL), (dict(E=0), moe.MOE_EINVAL),
    (dict(E=257, K=2), moe.MOE_EINVAL), (dict(D=0), moe.MOE_EINVAL), (dict(F=-1), moe.MOE_EINVAL),
    (dict(T=-1), moe.MOE_EINVAL), (dict(dtype=2), moe.MOE_ETYPE), (dict(out_dtype=7), moe.MOE_ETYPE),
    (dict(act=5), moe.MOE_ENOTSUP), (dict(T=2**31, K=2), moe.MOE_EINVAL),
])
def test_validation_codes(lib, kw, code):
    d = _desc(**kw)
    n = ctypes.c_size_t(0)
    assert lib.moe_workspace_bytes(ctypes.byref(d), ctypes.byref(n)) == code
    # nothing is dereferenced or launched on an error: bogus non-null pointers are safe here
    fake = 16
    assert moe.moe_forward(d, fake, fake, fake, fake, None, None, None, fake, fake, fake, None, None, fake,
                           1 << 40, None) == code
    assert moe.moe_dispatch(d, fake, fake, None, fake, fake, None, fake, fake, fake, fake, fake, 1 << 40,
                            None) == code


@pytest.mark.parametrize("desc_kw,rkw", [
    (dict(), dict(dynamic_threshold=-0.1)),
    (dict(), dict(dynamic_threshold=float("nan"))),
    (dict(norm_topk=0), dict(dynamic_threshold=0.2)),
    (dict(), dict(capacity_factor=-1.0)),
    (dict(), dict(capacity_factor=float("nan"))),
    (dict(), dict(capacity_factor=1.0, seq_len=5)),   # 5 does not divide T = 16
    (dict(), dict(seq_len=-4)),
])
def test_routing_validation(lib, desc_kw, rkw):
    d = _desc(**desc_kw)
    r = moe.MoeRouting(**rkw)
    fake = 16
    assert moe.moe_forward_routed(d, r, fake, fake, fake, fake, None, None, None, fake, fake, fake, None, None, fake,
                                  1 << 40, None) == moe.MOE_EINVAL
    assert moe.moe_dispatch_routed(d, r, fake, fake, None, fake, fake, None, fake, fake, fake, fake, fake, 1 << 40,
                                   None) == moe.MOE_EINVAL


def test_routing_options_off_is_plain_forward(lib):
    # a NULL routing pointer and an all-zero struct validate like moe_forward
    d = _desc(K=0)
    fake = 16
    for r in (None, moe.MoeRouting()):
        assert moe.moe_forward_routed(d, r, fake, fake, fake, fake, None, None, None, fake, fake, fake, None, None,
                                      fake, 1 << 40, None) == moe.MOE_EINVAL


def test_missing_pointers_and_small_workspace(lib):
    d = _desc()
    need = moe.moe_workspace_bytes(d)
    assert need > 0
    fake = 16
    assert moe.moe_forward(d, None, fake, fake, fake, None, None, None, fake, fake, fake, None, None, fake, need,
                           None) == moe.MOE_EINVAL
    assert moe.moe_forward(d, fake, fake, fake, fake, None, None, None, fake, fake, fake, None, None, fake, need - 1,
                           None) == moe.MOE_EWORKSPACE
    # x, gate_up_proj, down_proj and the workspace must start on 16-byte boundaries
    odd = fake + 2
    for i in (0, 2, 3, 12):
        args = [fake, fake, fake, fake, None, None, None, fake, fake, fake, None, None, fake]
        args[i] = odd
        assert moe.moe_forward(d, *args, need, None) == moe.MOE_EINVAL, i


def test_zero_tokens_is_a_no_op(lib):
    d = _desc(T=0)
    assert moe.moe_workspace_bytes(d) == 0
    assert moe.moe_forward(d, *([None] * 13), 0, None) == moe.MOE_OK


def test_workspace_grows_with_modes(lib):
    a = moe.moe_workspace_bytes(_desc(T=4096, D=512, F=2048))
    b = moe.moe_workspace_bytes(_desc(T=4096, D=512, F=2048, deterministic=1))
    c = moe.moe_workspace_bytes(_desc(T=4096, D=512, F=2048, out_dtype=1))
    assert b >= a + 4096 * 2 * 512 * 4       # per-(t,k) fp32 slots
    assert c >= a + 4096 * 512 * 4           # fp32 accumulation for a bf16 output
    # h (T*K rows of F) dominates: fp32 h for fp32 inputs
    assert a >= 4096 * 2 * 2048 * 4


def test_python_errors_map(lib):
    with pytest.raises(ValueError):
        moe._check(moe.MOE_EINVAL)
    with pytest.raises(NotImplementedError):
        moe._check(moe.MOE_ENOTSUP)
    with pytest.raises(TypeError):
        moe._check(moe.MOE_ETYPE)
    with pytest.raises(moe.MoEError):
        moe._check(moe.MOE_EDEVICE)


def test_bench_refuses_several_gpus():
    r = subprocess.run(["python3", os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_probes_validate_on_the_host(lib):
    # the FLOP count of a matrix-core probe launch: 8 waves x 8 chains of 32x32x16 MFMAs per round
    assert moe.moe_probe_mfma_flops(2, 3) == 2 * 8 * 3 * 8 * (2 * 32 * 32 * 16)
    assert moe.moe_probe_mfma_flops(0, 3) == 0
    einval = 1
    # rejected before any launch (no device needed)
    assert moe.moe_probe_mfma(0, 10, 4096, None) == einval
    assert moe.moe_probe_mfma(4, 0, 4096, None) == einval
    assert moe.moe_probe_mfma(4, 10, None, None) == einval
    assert moe.moe_probe_read(None, 1024, 4, 4096, None) == einval
    assert moe.moe_probe_read(4096, 1000, 4, 4096, None) == einval   # not a multiple of 16 bytes
    assert moe.moe_probe_read(4104, 1024, 4, 4096, None) == einval   # buffer not 16-byte aligned
    assert moe.moe_probe_read(4096, 1024, 0, 4096, None) == einval

