"""Host-side checks of the C ABI that run without a GPU.

The library must load, export every function include/kda_verify.h declares, and
reject every invalid argument before any HIP call. Pointers here are fake host
integers: only validation runs, nothing is launched.
"""
import ctypes
import os
import re

import pytest

import linear_attention_decode_kda_amd as kda
from linear_attention_decode_kda_amd import build as kbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda_verify.h")


@pytest.fixture(scope="module")
def lib():
    if kbuild.is_stale():
        kbuild.build()
    return kda.load()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert "kda_conv_verify_decode" in names and len(names) >= 7
    for name in names:
        assert hasattr(lib, name), f"{name} not exported"


def test_params_init_defaults(lib):
    p = kda.Params()
    lib.kda_verify_params_init(ctypes.byref(p), 3, 4, 2, 4, 128, 128)
    assert (p.N, p.T, p.H, p.HV, p.K, p.V) == (3, 4, 2, 4, 128, 128)
    assert p.in_dtype == kda.BF16 and p.gate_mode == kda.GATE_SOFTPLUS and p.variant == kda.VARIANT_AUTO
    assert p.lower_bound == -5.0 and p.softplus_beta == 1.0 and p.softplus_threshold == 20.0
    assert p.scale == 0.0 and p.l2norm_eps == pytest.approx(1e-6)


def test_workspace_bytes(lib):
    # one arrival counter per (sequence, q/k head) and the queue's two counters, in 256 B
    assert kda.workspace_bytes(kda.make_params(256, 4, 32, 32, 128, 128)) == 256 * 32 * 4 + 256
    assert kda.workspace_bytes(kda.make_params(3, 1, 2, 4, 128, 128)) == 256
    assert kda.workspace_bytes(kda.make_params(0, 1, 2, 4, 128, 128)) == 256
    assert kda.workspace_bytes(kda.make_params(3, 1, 2, 3, 128, 128)) == 0  # invalid: HV % H


def test_select_variant(lib):
    assert kda.select_variant(kda.make_params(256, 4, 32, 32, 128, 128)) == kda.VARIANT_LARGE
    assert kda.select_variant(kda.make_params(32, 4, 16, 16, 128, 128)) == kda.VARIANT_LARGE
    assert kda.select_variant(kda.make_params(4, 8, 16, 16, 128, 128)) == kda.VARIANT_SMALL
    assert kda.select_variant(kda.make_params(64, 3, 16, 32, 128, 128)) == kda.VARIANT_LARGE
    assert kda.select_variant(kda.make_params(512, 8, 16, 64, 128, 128)) == kda.VARIANT_LARGE
    assert kda.select_variant(kda.make_params(2, 2, 2, 2, 16, 16)) == kda.VARIANT_LARGE
    for v in (kda.VARIANT_SMALL, kda.VARIANT_LARGE):
        assert kda.select_variant(kda.make_params(1, 1, 1, 1, 128, 128, variant=v)) == v
    assert kda.select_variant(kda.make_params(1, 0, 1, 1, 128, 128)) == -2


def _fake_ptrs(p, ws_bytes=None):
    """Distinct, aligned, far-apart host integers standing in for device buffers."""
    ptrs = [(i + 1) << 40 for i in range(12)]
    return ptrs, (kda.workspace_bytes(p) if ws_bytes is None else ws_bytes)


def _validate(lib, p, ptrs, ws_bytes):
    return lib.kda_validate(ctypes.byref(p), *[ctypes.c_void_p(x) for x in ptrs], ws_bytes)


def test_validate_accepts_good_args(lib):
    for shape in [(256, 4, 32, 32, 128, 128), (2, 2, 2, 2, 16, 16), (3, 16, 1, 4, 64, 64)]:
        p = kda.make_params(*shape)
        ptrs, wsb = _fake_ptrs(p)
        assert _validate(lib, p, ptrs, wsb) == 0


@pytest.mark.parametrize("field,value,status", [
    ("T", 0, -2), ("T", 17, -2), ("N", -1, -2), ("H", 0, -2), ("HV", 3, -2),
    ("K", 32, -3), ("V", 64, -3), ("in_dtype", 7, -3), ("gate_mode", 2, -3), ("variant", 3, -3),
    ("softplus_beta", 0.0, -2), ("l2norm_eps", -1.0, -2),
])
def test_validate_rejects_bad_params(lib, field, value, status):
    p = kda.make_params(4, 4, 2, 4, 128, 128)
    ptrs, wsb = _fake_ptrs(p)
    setattr(p, field, value)
    assert _validate(lib, p, ptrs, wsb) == status
    # the launching entry point returns the same status without touching the GPU
    assert lib.kda_conv_verify_decode(ctypes.byref(p), *[ctypes.c_void_p(x) for x in ptrs], wsb, None) == status


def test_validate_pointer_errors(lib):
    p = kda.make_params(4, 4, 2, 4, 128, 128)
    ptrs, wsb = _fake_ptrs(p)
    for i in range(12):
        bad = list(ptrs)
        bad[i] = 0
        assert _validate(lib, p, bad, wsb) == -1, i
        bad[i] = ptrs[i] + 4
        assert _validate(lib, p, bad, wsb) == -4, i
    assert _validate(lib, p, ptrs, wsb - 4) == -5
    # an output overlapping an input or another output
    for out_i in (2, 8, 9, 10, 11):
        for other in range(12):
            if other == out_i:
                continue
            bad = list(ptrs)
            bad[out_i] = ptrs[other]
            assert _validate(lib, p, bad, wsb) == -7, (out_i, other)
    # inputs may alias each other (read only)
    bad = list(ptrs)
    bad[3] = ptrs[0]
    assert _validate(lib, p, bad, wsb) == 0


def test_zero_sequences_is_a_no_op(lib):
    p = kda.make_params(0, 4, 2, 4, 128, 128)
    null = [ctypes.c_void_p(0)] * 12
    assert lib.kda_validate(ctypes.byref(p), *null, 0) == 0
    assert lib.kda_conv_verify_decode(ctypes.byref(p), *null, 0, None) == 0


def test_noalloc_size_limit_and_params_checked_before_any_hip_call(lib):
    """The allocation-free entry point refuses shapes whose counters exceed its static
    scratch, and invalid params, on the host (no GPU here: a HIP call would fail)."""
    p = kda.make_params(4096, 1, 16, 16, 128, 128)  # 65536 + 2 counter words
    assert kda.workspace_bytes(p) > kda.NOALLOC_SCRATCH_BYTES
    fake = [ctypes.c_void_p((i + 1) << 40) for i in range(11)]
    assert lib.kda_conv_verify_decode_noalloc(ctypes.byref(p), *fake, None) == -8
    p = kda.make_params(4, 0, 2, 2, 128, 128)
    assert lib.kda_conv_verify_decode_noalloc(ctypes.byref(p), *fake, None) == -2
    p = kda.make_params(0, 4, 2, 2, 128, 128)  # an empty batch is a no-op
    assert lib.kda_conv_verify_decode_noalloc(ctypes.byref(p), *fake, None) == 0
    p = kda.make_params(4094, 1, 16, 16, 128, 128)  # 65504 + 2 words: fits
    assert kda.workspace_bytes(p) <= kda.NOALLOC_SCRATCH_BYTES
    assert "static scratch" in kda.lib_status_string(-8)


def test_status_strings(lib):
    for st in range(-7, 1):
        s = lib.kda_status_string(st).decode()
        assert s and s != "unknown status"
    assert lib.kda_status_string(-99).decode() == "unknown status"


def test_workspace_reset_argument_errors(lib):
    assert lib.kda_workspace_reset(None, 0, None) == 0
    assert lib.kda_workspace_reset(None, 256, None) == -1
    assert lib.kda_workspace_reset(ctypes.c_void_p(1 << 40), 6, None) == -4


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(kda, "_lib", None)
    monkeypatch.setattr(kda, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        kda.load()


def test_oracle_and_gpu_path_share_no_code():
    """The oracle and the HIP library neither import nor include each other."""
    pkg = os.path.join(ROOT, "linear_attention_decode_kda_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text and "kda_oracle" not in text, f
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith((".py", ".c", ".h")):
            text = open(os.path.join(ROOT, "oracle", f)).read()
            assert "linear_attention_decode_kda_amd" not in text and "kda_verify" not in text, f


def _pooled_raw(lib, p, pd, ptrs, wsb):
    return lib.kda_conv_verify_decode_pooled(ctypes.byref(p), ctypes.byref(pd) if pd is not None else None,
                                             *[ctypes.c_void_p(x) for x in ptrs], wsb, None)


def test_pool_descriptor_validation(lib):
    """Pool errors are caught on the host before any launch (fake pointers, no GPU)."""
    p = kda.make_params(4, 4, 2, 4, 128, 128)
    p.T = 0  # invalid params first: nothing reaches the pools
    ptrs, wsb = _fake_ptrs(kda.make_params(4, 4, 2, 4, 128, 128))
    assert _pooled_raw(lib, p, kda.PoolDesc(), ptrs, wsb) == -2
    p = kda.make_params(4, 4, 2, 4, 128, 128)
    pd = kda.PoolDesc()
    pd.conv_state_slots, pd.state_slots, pd.intermediate_slots = 4, 0, 4
    assert _pooled_raw(lib, p, pd, ptrs, wsb) == -2  # an empty pool
    pd.state_slots = 3
    assert _pooled_raw(lib, p, pd, ptrs, wsb) == -2  # identity rows need N slots
    pd.state_slots = 3
    pd.cache_indices = (13 << 40) + 2
    assert _pooled_raw(lib, p, pd, ptrs, wsb) == -4  # misaligned index array
    pd.cache_indices = ptrs[9]
    assert _pooled_raw(lib, p, pd, ptrs, wsb) == -7  # index array inside inter_ssm (written)


def test_commit_validation(lib):
    p = kda.make_params(4, 4, 2, 4, 128, 128)
    ptrs = [(i + 1) << 40 for i in range(5)]
    args = lambda q: [ctypes.c_void_p(x) for x in q]  # noqa: E731
    bad = list(ptrs)
    bad[0] = 0
    assert lib.kda_verify_commit(ctypes.byref(p), None, *args(bad), None) == -1
    bad = list(ptrs)
    bad[3] = ptrs[1]  # state written over inter_ssm
    assert lib.kda_verify_commit(ctypes.byref(p), None, *args(bad), None) == -7
    p0 = kda.make_params(0, 4, 2, 4, 128, 128)
    assert lib.kda_verify_commit(ctypes.byref(p0), None, *args([0] * 5), None) == 0
    bad = list(ptrs)
    bad[0] += 2  # misaligned accepted lengths
    assert lib.kda_verify_commit(ctypes.byref(p), None, *args(bad), None) == -4
    bad = list(ptrs)
    bad[0] = ptrs[3] + 64  # accepted lengths inside the state pool the commit writes
    assert lib.kda_verify_commit(ctypes.byref(p), None, *args(bad), None) == -7
    bad = list(ptrs)
    bad[4] = ptrs[3]  # conv_state and state written over one another
    assert lib.kda_verify_commit(ctypes.byref(p), None, *args(bad), None) == -7
    pd = kda.PoolDesc()
    pd.conv_state_slots, pd.state_slots, pd.intermediate_slots = 4, 3, 4
    assert lib.kda_verify_commit(ctypes.byref(p), ctypes.byref(pd), *args(ptrs), None) == -2  # identity needs N rows
    pd.state_slots = 8
    pd.cache_indices = ptrs[3] + 16  # an index array inside the state pool, which the commit writes
    assert lib.kda_verify_commit(ctypes.byref(p), ctypes.byref(pd), *args(ptrs), None) == -7
    bad_p = kda.make_params(4, 4, 2, 4, 128, 128)
    bad_p.HV = 5
    assert lib.kda_verify_commit(ctypes.byref(bad_p), None, *args(ptrs), None) == -2


def test_commit_contract_is_stated_in_the_header():
    """Distinct written rows among committed sequences are the caller's contract (the
    index arrays are device memory the host never reads); the header says so."""
    src = open(HEADER).read()
    head = src[src.index("kda_status kda_verify_commit") - 2200:src.index("kda_status kda_verify_commit")]
    assert "must be distinct among the sequences it commits" in head
    assert "is not checked" in head and "race" in head


def test_tuning_overrides(lib):
    p = kda.make_params(256, 4, 32, 32, 128, 128, tile_columns=128)
    assert kda.select_variant(p) == kda.VARIANT_LARGE
    p = kda.make_params(8, 4, 2, 2, 128, 128, tile_columns=32, variant=kda.VARIANT_LARGE)
    assert kda.select_variant(p) == kda.VARIANT_SMALL  # the tile override wins
    for bad in (dict(tile_columns=48), dict(store_policy=3), dict(max_wg_per_cu=3), dict(max_wg_per_cu=7),
                dict(max_wg_per_cu=-1), dict(column_groups=3), dict(column_groups=8),
                dict(tile_columns=64, column_groups=2), dict(variant=kda.VARIANT_SMALL, column_groups=4),
                dict(dtype="f32", T=12, column_groups=2), dict(schedule=4), dict(schedule=-1),
                dict(schedule=3, T=9), dict(schedule=3, column_groups=2), dict(schedule=3, max_wg_per_cu=2),
                dict(schedule=3, tile_columns=64), dict(schedule=3, variant=kda.VARIANT_SMALL),
                dict(prefetch=3), dict(prefetch=-1),
                dict(tile_columns=64, schedule=2), dict(variant=kda.VARIANT_SMALL, schedule=2),
                dict(dtype="f32", T=12, schedule=2), dict(unit_order=3), dict(unit_order=-1)):
        kw = dict(bad)
        p = kda.make_params(8, kw.pop("T", 4), 2, 2, 128, 128, **kw)
        ptrs, wsb = _fake_ptrs(p)
        assert _validate(lib, p, ptrs, wsb) == -3, bad
    for good in (1, 2, 4, 6, 8):
        p = kda.make_params(8, 4, 2, 2, 128, 128, max_wg_per_cu=good)
        ptrs, wsb = _fake_ptrs(p)
        assert _validate(lib, p, ptrs, wsb) == 0
    p = kda.make_params(8, 4, 2, 2, 64, 64, tile_columns=64)  # overrides exist for K = V = 128 only
    ptrs, wsb = _fake_ptrs(p)
    assert _validate(lib, p, ptrs, wsb) == -3
    p = kda.make_params(8, 4, 2, 2, 64, 64, variant=kda.VARIANT_SMALL, schedule=2)  # the queue takes whole V
    ptrs, wsb = _fake_ptrs(p)
    assert _validate(lib, p, ptrs, wsb) == -3
    for good in (dict(schedule=1), dict(schedule=2), dict(schedule=2, max_wg_per_cu=2, column_groups=4)):
        p = kda.make_params(8, 4, 2, 2, 128, 128, **good)
        ptrs, wsb = _fake_ptrs(p)
        assert _validate(lib, p, ptrs, wsb) == 0, good


# launches a kernel exists for at K = V = 128: (columns per workgroup, column groups)
BUILT_128 = {(128, 1), (128, 2), (128, 4), (64, 1), (32, 1)}


def test_every_accepted_override_names_a_built_launch(lib):
    """Any combination of overrides that validates resolves to a launch some kernel
    implements: column groups split whole-V workgroups only, so asking for groups without a
    tile takes whole V even where AUTO's own tile is narrower (the 32-column split of a
    one-sequence call)."""
    p = kda.make_params(1, 4, 8, 8, 128, 128)
    assert kda.select_launch(p)["tile_columns"] == 32
    p = kda.make_params(1, 4, 8, 8, 128, 128, column_groups=2)
    assert tuple(kda.select_launch(p).values()) == (128, 1, 0, 2, 1, 2, 0)
    for N, T, H, HV, dt in ((64, 2, 16, 32, "bf16"), (1, 4, 8, 8, "bf16"), (512, 8, 16, 64, "bf16"),
                            (8, 12, 2, 2, "f32"), (32, 1, 16, 16, "bf16"), (128, 3, 16, 32, "bf16")):
        for tile in (0, 32, 64, 128):
            for groups in (0, 1, 2, 4):
                for sched in (0, 1, 2, 3):
                    for variant in (kda.VARIANT_AUTO, kda.VARIANT_SMALL, kda.VARIANT_LARGE):
                        p = kda.make_params(N, T, H, HV, 128, 128, dtype=dt, tile_columns=tile, column_groups=groups,
                                            schedule=sched, variant=variant)
                        ptrs, wsb = _fake_ptrs(p)
                        if _validate(lib, p, ptrs, wsb) != 0:
                            continue
                        got = kda.select_launch(p)
                        key = (got["tile_columns"], got["column_groups"])
                        assert key in BUILT_128, (N, T, H, HV, dt, tile, groups, sched, variant, got)
                        if dt == "f32" and T > 8:
                            assert got["tile_columns"] < 128
                        if got["schedule"] >= 2:
                            assert got["tile_columns"] == 128
                        if got["schedule"] == 3:  # the stream kernel: one group, T <= 8
                            assert got["column_groups"] == 1 and T <= 8 and got["max_wg_per_cu"] == 1
                            assert got["prefetch"] in (1, 2)


def test_prepared_call_checks_arguments_once():
    """PreparedVerify runs the same argument checks as the plain call (no GPU needed to
    see a rejection: CPU tensors are refused before anything reaches the library)."""
    import torch
    from linear_attention_decode_kda_amd import synth
    w = synth.WORKLOADS["tiny"]
    inp = synth.make_inputs(w)
    out = {"o": torch.empty(w.N, w.T, w.HV, w.V), "inter_ssm": torch.empty(w.N, w.T, w.HV, w.K, w.V),
           "conv_window": torch.empty(w.N, w.T, w.C, 3)}
    p = kda.params_for(w)
    with pytest.raises(ValueError, match="GPU device"):
        kda.PreparedVerify(p, inp, out, torch.zeros(256, dtype=torch.uint8))


def test_select_launch_follows_the_dispatch_rule(lib):
    """The AUTO rule (tile, stores, workgroups-per-CU cap, column groups, schedule: 1 grid,
    2 queue, 3 stream) on the named workloads and at the edges of its five buckets, and the
    overrides winning over it."""
    L = lambda *shape, **kw: tuple(kda.select_launch(kda.make_params(*shape, **kw)).values())[:5]
    assert L(2, 2, 2, 2, 16, 16) == (16, 1, 0, 1, 1)            # tiny: the only K = V = 16 tile
    assert L(32, 4, 16, 16, 128, 128) == (128, 1, 0, 1, 1)       # small batch: 512 units, T = 4
    assert L(64, 3, 16, 32, 128, 128) == (128, 2, 1, 1, 3)       # GVA: 2048 units, T = 3
    assert L(256, 4, 32, 32, 128, 128) == (128, 2, 1, 1, 3)      # large batch: 8192 units
    assert L(512, 8, 16, 64, 128, 128) == (128, 2, 1, 1, 3)      # max bandwidth: 32768 units, T = 8
    # 1. <= 64 units, and <= 128 at T = 2: the 32-column split
    assert L(1, 4, 8, 8, 128, 128) == (32, 1, 0, 1, 1)
    assert L(4, 4, 16, 16, 128, 128) == (32, 1, 0, 1, 1)
    assert L(8, 2, 16, 16, 128, 128) == (32, 1, 0, 1, 1)
    # ... and four column groups up to 128 units
    assert L(8, 4, 16, 16, 128, 128) == (128, 1, 0, 4, 1)
    assert L(5, 7, 4, 20, 128, 128) == (128, 1, 0, 4, 1)
    # 2. 129-512 units, no cap: groups ...
    assert L(8, 1, 32, 32, 128, 128) == (128, 1, 0, 4, 1)        # T = 1: four up to 256 units ...
    assert L(9, 1, 32, 32, 128, 128) == (128, 2, 0, 1, 1)        # ... one beyond
    assert L(12, 4, 32, 32, 128, 128) == (128, 1, 0, 2, 1)       # two below 448 ...
    assert L(14, 4, 32, 32, 128, 128) == (128, 1, 0, 1, 1)       # ... one from 448
    assert L(7, 3, 16, 32, 128, 128) == (128, 2, 0, 2, 1)        # odd T: two below 256 units ...
    assert L(8, 3, 32, 32, 128, 128) == (128, 2, 0, 1, 1)        # ... one from 256
    assert L(13, 7, 32, 32, 128, 128) == (128, 2, 0, 1, 1)
    assert L(8, 6, 16, 32, 128, 128) == (128, 2, 0, 2, 1)        # even T >= 6: device-scope stores
    assert L(16, 8, 16, 32, 128, 128) == (128, 2, 0, 1, 1)
    assert L(16, 2, 16, 16, 128, 128) == (128, 1, 0, 2, 1)       # T = 2 and 4: streaming stores
    # 3. the uncapped grid: below 1024 units, below 1280 units at T = 2, below 3072 at T = 1
    assert L(24, 4, 32, 32, 128, 128) == (128, 2, 0, 1, 1)
    assert L(31, 8, 16, 32, 128, 128) == (128, 2, 0, 1, 1)
    assert L(64, 1, 32, 32, 128, 128) == (128, 2, 0, 1, 1)
    assert L(95, 1, 32, 32, 128, 128) == (128, 2, 0, 1, 1)
    assert L(96, 1, 32, 32, 128, 128) == (128, 2, 1, 1, 3)      # T = 1 from 3072 units: the stream
    assert L(512, 1, 16, 64, 128, 128) == (128, 2, 1, 1, 3)
    assert L(39, 2, 32, 32, 128, 128) == (128, 2, 0, 1, 1)       # 1248 units
    assert L(40, 2, 32, 32, 128, 128) == (128, 2, 1, 1, 3)       # 1280 units: the stream
    assert L(63, 2, 32, 32, 128, 128) == (128, 2, 1, 1, 3)
    # 4. two per CU below 1280 units at T = 3, 4
    assert L(32, 3, 32, 32, 128, 128) == (128, 2, 2, 1, 1)
    assert L(39, 4, 16, 32, 128, 128) == (128, 2, 2, 1, 1)       # 1248 units
    assert L(40, 4, 16, 32, 128, 128) == (128, 2, 1, 1, 3)       # 1280 units: the stream
    # 5. the stream, one per CU: from 1280 units at T = 2-4, from 1024 at T >= 5; the
    # queue above T = 8
    assert L(64, 2, 16, 32, 128, 128) == (128, 2, 1, 1, 3)
    assert L(64, 3, 32, 32, 128, 128) == (128, 2, 1, 1, 3)
    assert L(32, 5, 16, 32, 128, 128) == (128, 2, 1, 1, 3)
    assert L(31, 8, 32, 32, 128, 128) == (128, 2, 0, 1, 1)
    assert L(32, 8, 32, 32, 128, 128) == (128, 2, 1, 1, 3)
    assert L(1024, 16, 8, 8, 128, 128) == (128, 2, 1, 1, 2)
    assert L(128, 9, 8, 16, 128, 128) == (128, 2, 1, 1, 2)
    assert L(64, 8, 16, 32, 128, 128, dtype="f32") == (128, 2, 1, 1, 3)
    # the stream's state prefetch: at the start up to 65536 snapshot tiles per call, after the
    # conv beyond; the override wins
    F = lambda *shape, **kw: kda.select_launch(kda.make_params(*shape, **kw))["prefetch"]
    assert F(64, 3, 16, 32, 128, 128) == 2 and F(256, 4, 32, 32, 128, 128) == 2
    assert F(256, 8, 32, 32, 128, 128) == 2                      # 65536 tiles
    assert F(512, 8, 16, 64, 128, 128) == 1 and F(512, 4, 16, 64, 128, 128) == 1
    assert F(256, 2, 32, 32, 128, 128) == 2 and F(1024, 2, 64, 64, 128, 128) == 1   # T = 2
    assert F(256, 4, 32, 32, 128, 128, prefetch=1) == 1 and F(512, 8, 16, 64, 128, 128, prefetch=2) == 2
    assert F(32, 4, 16, 16, 128, 128) == 0 and F(1024, 16, 8, 8, 128, 128) == 0  # not the stream
    # overrides
    assert L(256, 4, 32, 32, 128, 128, tile_columns=32, store_policy=2, max_wg_per_cu=6) == (32, 2, 6, 1, 1)
    assert L(256, 4, 32, 32, 128, 128, tile_columns=32) == (32, 2, 0, 1, 1)   # the AUTO cap goes with its tile
    assert L(32, 4, 32, 32, 128, 128, tile_columns=128) == (128, 2, 0, 1, 1)  # caller's tile: no AUTO cap
    assert L(32, 4, 32, 32, 128, 128, max_wg_per_cu=8) == (128, 2, 0, 1, 1)   # 8: explicitly none
    assert L(32, 4, 32, 32, 128, 128, tile_columns=128, max_wg_per_cu=2) == (128, 2, 2, 1, 1)
    assert L(32, 4, 32, 32, 128, 128, variant=kda.VARIANT_SMALL) == (32, 2, 0, 1, 1)
    assert L(32, 4, 32, 32, 128, 128, variant=kda.VARIANT_LARGE) == (128, 2, 0, 1, 1)
    assert L(32, 4, 32, 32, 128, 128, store_policy=1) == (128, 1, 2, 1, 1)
    assert L(32, 4, 32, 32, 128, 128, column_groups=4) == (128, 2, 2, 4, 1)
    assert L(3, 16, 1, 4, 64, 64, max_wg_per_cu=2) == (64, 1, 2, 1, 1)
    assert L(256, 4, 32, 32, 128, 128, schedule=1) == (128, 2, 1, 1, 1)      # the grid, AUTO cap kept
    assert L(256, 4, 32, 32, 128, 128, schedule=2) == (128, 2, 1, 1, 2)      # the queue, AUTO cap kept
    assert L(32, 4, 32, 32, 128, 128, schedule=2) == (128, 2, 2, 1, 2)
    assert L(32, 4, 32, 32, 128, 128, schedule=3) == (128, 2, 1, 1, 3)      # the stream: one per CU
    assert L(16, 2, 16, 16, 128, 128, schedule=3) == (128, 1, 1, 1, 3)      # ... and one group
    assert L(1, 4, 8, 8, 128, 128, schedule=3) == (128, 1, 1, 1, 3)
    # a caller's groups or cap take the AUTO stream back to the queue, which honours them
    assert L(256, 4, 32, 32, 128, 128, column_groups=2) == (128, 2, 1, 2, 2)
    assert L(256, 4, 32, 32, 128, 128, max_wg_per_cu=8) == (128, 2, 0, 1, 2)
    assert L(256, 4, 32, 32, 128, 128, max_wg_per_cu=1) == (128, 2, 1, 1, 3)
    assert L(1, 4, 8, 8, 128, 128, schedule=2) == (128, 1, 0, 1, 2)          # the queue takes whole V
    assert L(8, 4, 16, 16, 128, 128, tile_columns=128) == (128, 1, 0, 1, 1)  # caller's tile: one group
    assert L(256, 4, 32, 32, 128, 128, tile_columns=128, schedule=2) == (128, 2, 0, 1, 2)
    assert L(256, 4, 32, 32, 128, 128, tile_columns=128) == (128, 2, 0, 1, 1)  # caller's tile: the grid
    assert L(3, 16, 1, 4, 64, 64, schedule=2) == (64, 1, 0, 1, 2)
    # fp32 at T > 8: two 64-column workgroups, one group each, on the grid
    assert L(64, 9, 8, 16, 128, 128, dtype="f32") == (64, 2, 1, 1, 1)
    assert L(512, 9, 32, 32, 128, 128, dtype="f32") == (64, 2, 1, 1, 1)
    assert kda.make_params(1, 0, 1, 1, 128, 128) and lib.kda_select_launch(
        ctypes.byref(kda.make_params(1, 0, 1, 1, 128, 128)), None, None, None, None, None, None, None) == -2
    # unit order: pairs for whole-V grids without a cap (every workgroup resident at once),
    # XCD ranges for capped grids, the 32-column split and the queue; the override wins
    O = lambda *shape, **kw: kda.select_launch(kda.make_params(*shape, **kw))["unit_order"]
    assert O(32, 4, 16, 16, 128, 128) == 2                      # small batch
    assert O(12, 4, 32, 32, 128, 128) == 2 and O(8, 4, 16, 16, 128, 128) == 2
    assert O(32, 3, 32, 32, 128, 128) == 1                      # capped grid
    assert O(24, 4, 32, 32, 128, 128) == 2                      # uncapped grid of 768 units
    assert O(256, 4, 32, 32, 128, 128) == 1 and O(1, 4, 8, 8, 128, 128) == 1
    assert O(256, 4, 32, 32, 128, 128, schedule=2) == 1
    assert O(2, 2, 2, 2, 16, 16) == 2                           # K = V = 16: whole V, no cap
    assert O(32, 4, 16, 16, 128, 128, unit_order=1) == 1 and O(256, 4, 32, 32, 128, 128, unit_order=2) == 2
    G = lambda *shape, **kw: kda.select_launch(kda.make_params(*shape, **kw))["column_groups"]
    assert G(256, 4, 32, 32, 128, 128, column_groups=4) == 4
    assert G(256, 4, 32, 32, 128, 128, tile_columns=128) == 1     # caller's tile: one group unless asked
    assert G(256, 4, 32, 32, 128, 128, tile_columns=128, column_groups=2) == 2
