"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, and rejects bad arguments on the host before any launch."""
import ctypes
import glob
import os
import re
import subprocess

import pytest

import sparse_mixture_experts_02_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


def declared_functions():
    names = set()
    for h in HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(moe_\w+)\s*\(", src, flags=re.M))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moe.LIB_PATH):
        pytest.fail("libmoe.so is not built (run python -m sparse_mixture_experts_02_amd.build)")
    return moe.load_library()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("moe_forward", "moe_forward_timed", "moe_forward_routed", "moe_dispatch", "moe_dispatch_routed",
              "moe_workspace_bytes", "moe_status_string", "moe_abi_version", "moe_probe_mfma", "moe_probe_read"):
        assert n in names
    # the layer's header carries the layer only; the probes have their own
    layer = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "moe.h")).read(), flags=re.S)
    assert "moe_probe" not in layer


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
    # the FLOP count of a matrix-core probe launch: 8 waves x 8 chains of 16x16x32 MFMAs per round
    assert moe.moe_probe_mfma_flops(2, 3) == 2 * 8 * 3 * 8 * (2 * 16 * 16 * 32)
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



@pytest.mark.parametrize("act,which,shape", [
    ("silu", "router_bias", (9,)), ("silu", "router_bias", (8, 1)),
    ("silu", "up_bias", (8, 128)),          # an (E, F) bias on a SwiGLU layer: the up half would be read past it
    ("silu", "up_bias", (256,)),            # one bias shared by the experts
    ("relu", "up_bias", (8, 256)),
    ("silu", "down_bias", (8, 128)), ("relu", "down_bias", (64,)),
])
def test_bias_shapes_are_checked_before_any_pointer_is_passed(act, which, shape):
    """The kernels index the router bias as (E), the up bias as (E, G*F) and
    the down bias as (E, D): the binding refuses anything else with a
    ValueError naming the bias (on CPU tensors the check comes before the
    device check, so no GPU is needed)."""
    torch = pytest.importorskip("torch")
    E, D, F = 8, 64, 128
    G = 1 if act == "relu" else 2
    x = torch.zeros(5, D)
    args = (x, torch.zeros(E, D), torch.zeros(E, G * F, D), torch.zeros(E, D, F))
    good = dict(router_bias=torch.zeros(E), up_bias=torch.zeros(E, G * F), down_bias=torch.zeros(E, D))
    with pytest.raises(ValueError, match="ROCm device"):
        moe.forward(*args, top_k=2, act=act, **good)
    bad = dict(good, **{which: torch.zeros(*shape)})
    with pytest.raises(ValueError, match=which):
        moe.forward(*args, top_k=2, act=act, **bad)


def test_noalloc_refuses_oversize_before_any_launch(lib):
    # workspace of the Mixtral-shaped prefill (~0.75 GB) is above the fixed array
    d = _desc(T=8192, D=4096, F=14336, E=8, K=2, dtype=1, deterministic=1)
    assert moe.moe_workspace_bytes(d) > moe.MOE_NOALLOC_MAX_BYTES
    fake = 256
    assert moe.moe_forward_noalloc(d, fake, fake, fake, fake, None, None, None, fake, fake, fake, None, None,
                                   None) == moe.MOE_EWORKSPACE
    # argument errors come first, as for moe_forward
    assert moe.moe_forward_noalloc(_desc(K=0), fake, fake, fake, fake, None, None, None, fake, fake, fake, None,
                                   None, None) == moe.MOE_EINVAL
    assert moe.moe_forward_noalloc(_desc(T=0), *([None] * 12), None) == moe.MOE_OK


@pytest.mark.parametrize("kw,g1,g2", [
    # the Mixtral-shaped prefill: 2048 rows per expert -> 256-row tiles with tail strips
    (dict(T=8192, D=4096, F=14336, E=8, K=2, dtype=1), "direct_m256_tail", "direct_m256_tail"),
    # the 64-token decode batch: 16 rows per expert, bf16, K a multiple of 512 -> weight streaming
    # on narrow tiles: gate_up 1792 items (7 whole rounds of 256 CUs), down 256 items (one round,
    # no better than 128 wide tiles cut in two along K, so no K split and no fix-up)
    (dict(T=64, D=4096, F=14336, E=8, K=2, dtype=1), "stream_m32_narrow", "stream_m32_narrow"),
    (dict(T=64, D=4096, F=14336, E=8, K=2, dtype=1, deterministic=1), "stream_m32_narrow", "stream_m32_narrow"),
    # one token: 2 experts x 16 down column tiles of 256 -> wide tiles cut in 8 along K
    # (deterministic mode only; the atomic combine never splits)
    (dict(T=1, D=4096, F=14336, E=8, K=2, dtype=1, deterministic=1), "stream_m32_narrow", "stream_m32"),
    (dict(T=1, D=4096, F=14336, E=8, K=2, dtype=1, deterministic=0), "stream_m32_narrow", "stream_m32_narrow"),
    # 128 and 200 tokens: 32 and 50 rows per expert -> the 64-row narrow streaming tile, which
    # reads each expert's weights once for up to 64 rows; 100 tokens (25 rows) keeps 32-row tiles
    (dict(T=128, D=4096, F=14336, E=8, K=2, dtype=1, deterministic=1), "stream_m64_narrow", "stream_m64_narrow"),
    (dict(T=200, D=4096, F=14336, E=8, K=2, dtype=1, deterministic=0), "stream_m64_narrow", "stream_m64_narrow"),
    (dict(T=100, D=4096, F=14336, E=8, K=2, dtype=1, deterministic=1), "stream_m32_narrow", "stream_m32_narrow"),
    # the same in fp32: the direct 32-row tiles
    (dict(T=64, D=4096, F=14336, E=8, K=2, dtype=0), "direct_m32", "direct_m32"),
    # gate_up contracts over D = 768 (not a multiple of 512), down over F = 1024
    (dict(T=64, D=768, F=1024, E=8, K=2, dtype=1), "direct_m32", "stream_m32_narrow"),
    # gate_up's 1040 output columns are a multiple of 16 but not of 32; down
    # contracts over 1040 (not whole 128-byte stages) -> the generic kernel
    (dict(T=64, D=1024, F=1040, E=8, K=2, dtype=1), "direct_m32", "generic_m64"),
    # the 128-expert layer: 1024 rows per expert -> 256-row tiles
    (dict(T=16384, D=2048, F=768, E=128, K=8, dtype=1), "direct_m256_tail", "direct_m256_tail"),
    # bf16 from 58 rows per expert: the 256-row ping-pong tile (250 rows per expert here; 60 and
    # 64 at 240 and 256 tokens, where 220 tokens, 55 rows, still streams on 64-row tiles)
    (dict(T=1000, D=512, F=1024, E=8, K=2, dtype=1), "direct_m256_tail", "direct_m256_tail"),
    (dict(T=256, D=4096, F=14336, E=8, K=2, dtype=1), "direct_m256_tail", "direct_m256_tail"),
    (dict(T=240, D=4096, F=14336, E=8, K=2, dtype=1), "direct_m256_tail", "direct_m256_tail"),
    (dict(T=220, D=4096, F=14336, E=8, K=2, dtype=1), "stream_m64_narrow", "stream_m64_narrow"),
    # fp32 too: 256-row tiles from 58 rows per expert
    (dict(T=1000, D=512, F=1024, E=8, K=2, dtype=0), "direct_m256_tail", "direct_m256_tail"),
    # K not filling 128-byte stages -> the generic kernel
    (dict(T=1000, D=40, F=48, E=8, K=2, dtype=0), "generic_m64", "generic_m64"),
])
def test_gemm_plan_picks_the_kernel_for_the_shape(lib, kw, g1, g2):
    plan = moe.moe_gemm_plan(_desc(**kw))
    assert plan["gate_up"]["variant"] == g1 and plan["down"]["variant"] == g2, plan
    for name, N in (("gate_up", kw["F"]), ("down", kw["D"])):
        p = plan[name]
        assert p["col_tiles"] == -(-N // p["cols"])
        assert p["max_items"] >= p["col_tiles"]


def test_gemm_plan_k_split_rules(lib):
    # wide streaming tiles: 4 experts x 8 gate_up column tiles = 32 items, cut
    # into 8 K parts (8 chunks of 512 each); the narrow tiles would fill only
    # 64 of 256 CUs
    p = moe.moe_gemm_plan(_desc(T=16, D=4096, F=1024, E=4, K=2, dtype=1, deterministic=1))
    assert p["gate_up"]["variant"] == "stream_m32" and p["gate_up"]["k_split"]
    # the down GEMM splits only in the deterministic mode
    det = moe.moe_gemm_plan(_desc(T=1, D=4096, F=14336, E=8, K=2, dtype=1, deterministic=1))
    atom = moe.moe_gemm_plan(_desc(T=1, D=4096, F=14336, E=8, K=2, dtype=1, deterministic=0))
    assert det["down"]["k_split"] and not atom["down"]["k_split"]
    # a 3584-long contraction has 7 chunks of 512: never split -> narrow tiles
    short = moe.moe_gemm_plan(_desc(T=16, D=3584, F=1024, E=4, K=2, dtype=1, deterministic=1))
    assert short["gate_up"]["variant"] == "stream_m32_narrow" and not short["gate_up"]["k_split"]
    # the narrow tiles never split
    for q in (det, atom, short):
        for g in ("gate_up", "down"):
            assert not (q[g]["variant"] == "stream_m32_narrow" and q[g]["k_split"])
    with pytest.raises(ValueError):
        moe.moe_gemm_plan(_desc(K=0))
