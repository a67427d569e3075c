"""Host-side tests of libfd (no GPU needed): the shared library loads, exports
every function include/fd.h declares, sizes its workspace as documented,
plans split counts by its stated rule, and rejects bad arguments before
launching anything."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fd.h")

fd = pytest.importorskip("decode_attention_09_amd")


def _lib():
    try:
        return fd.load_library()
    except RuntimeError as e:  # pragma: no cover - only when not built
        pytest.fail(f"libfd.so must be built before the tests: {e}")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fd_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("fd_plan_splits", "fd_workspace_bytes", "fd_decode_attention", "fd_decode_split",
              "fd_decode_combine", "fd_status_string", "fd_last_error", "fd_set_kernel_path",
              "fd_workspace_bytes_unnorm", "fd_decode_split_unnorm", "fd_decode_combine_unnorm",
              "fd_decode_attention_unnorm", "fd_set_schedule", "fd_decode_attention_noalloc", "fd_set_combine",
              "fd_plan_schedule", "fd_plan_time_us"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = _lib()
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_python_binding_has_the_c_names():
    for n in declared_functions():
        assert callable(getattr(fd, n)), n


def test_status_strings():
    assert fd.fd_status_string(0) == "ok"
    for s in (1, 2, 3, 4, 99):
        assert isinstance(fd.fd_status_string(s), str) and fd.fd_status_string(s)
    assert fd.fd_last_error() == ""


@pytest.mark.parametrize("B,H,D,ns", [(1, 8, 128, 7), (4, 32, 16, 16), (32, 28, 128, 8),
                                      (3, 5, 64, 1000)])
def test_workspace_bytes_layout(B, H, D, ns):
    n = fd.fd_workspace_bytes(B, H, ns, D)
    opart = B * H * ns * D * 4
    lse_off = (opart + 255) // 256 * 256
    ctl_off = lse_off + (B * ns * H * 4 + 255) // 256 * 256
    # control block: the queue's claim counter (256 B), then B*H arrival
    # counters of fused calls padded to 256 B, then the steal schedule's
    # 4096 64-bit share words
    assert n == ctl_off + 256 + (B * H * 4 + 255) // 256 * 256 + 4096 * 8


@pytest.mark.parametrize("B,H,D,ns", [(1, 8, 128, 7), (4, 32, 16, 16), (3, 5, 64, 1000)])
def test_workspace_bytes_unnorm_layout(B, H, D, ns):
    # ACC [B,H,ns,D], then M [B,H,ns] and L [B,H,ns], each at a 256-B boundary
    n = fd.fd_workspace_bytes_unnorm(B, H, ns, D)
    rows = B * H * ns
    off_m = (rows * D * 4 + 255) // 256 * 256
    off_l = off_m + (rows * 4 + 255) // 256 * 256
    assert n == off_l + rows * 4
    assert fd.fd_workspace_bytes_unnorm(0, H, ns, D) == 0
    assert fd.fd_workspace_bytes_unnorm(B, H, ns, 96) == 0


def test_workspace_bytes_rejects_bad_sizes():
    assert fd.fd_workspace_bytes(0, 8, 4, 128) == 0
    assert fd.fd_workspace_bytes(1, 8, 4, 100) == 0
    assert fd.fd_workspace_bytes(1, 8, 0, 128) == 0
    assert fd.fd_workspace_bytes(1, 8, fd.FD_MAX_SPLITS + 1, 128) == 0


# ----------------------------------------------------------------- planner --
def plan(B, H, Hkv, D, lens, cus=256, max_splits=0, dtype=fd.FD_F16):
    return fd.fd_plan_splits(B, H, Hkv, D, dtype, lens, cus, max_splits)


def test_planner_never_creates_an_empty_split():
    # decode_attention_splitkv.py: every split needs >= 1 key, else fall back
    for lens in ([1], [3, 4096], [7, 100000], [64] * 32, [1, 1, 1]):
        ns = plan(len(lens), 8, 1, 128, lens)
        assert 1 <= ns <= min(lens)


def test_planner_rejects_empty_sequences():
    with pytest.raises(fd.FdError) as e:
        plan(2, 8, 1, 128, [5, 0])
    assert e.value.status == 3


def test_planner_keeps_256_keys_per_split():
    for L in (256, 1000, 4096, 65536, 131072):
        ns = plan(1, 32, 8, 128, [L])
        assert ns <= max(1, math.ceil(L / 256))


def test_planner_no_split_when_one_pass_fills_the_device():
    # 256 x 2 KV heads = 512 workgroups already give every one of 256 CUs work
    assert plan(256, 16, 2, 128, [256] * 256) == 1


def test_planner_splits_a_single_long_sequence():
    # 1 sequence x 8 KV heads: one workgroup per head leaves the device idle;
    # the split count fills the 256 CUs with whole rounds of workgroups
    ns = plan(1, 32, 8, 128, [131072])
    wgs = 8 * ns
    assert ns >= 16 and wgs % 256 == 0


def test_planner_quantises_to_the_cu_count():
    # measured on MI355X: 16/2 heads, batch 8 x 8192 keys is fastest at 16
    # splits (256 workgroups), batch 1 x 65536 at 128 (256 workgroups)
    assert plan(8, 16, 2, 128, [8192] * 8) == 16
    assert plan(1, 16, 2, 128, [65536]) == 128


def test_planner_spreads_unequal_lengths():
    # varlen batch: more, shorter splits than the uniform rule would take,
    # so the longest sequence does not set the tail
    import numpy as np
    lens = np.random.default_rng(0).integers(64, 32769, 32).tolist()
    ns = plan(32, 28, 4, 128, lens)
    assert ns >= 8 and ns <= min(lens)
    assert plan(32, 28, 4, 128, [max(lens)] * 32) <= ns


def test_planner_wave_quantisation_example():
    # 04_flash_decoding.py, demo 4: batch 64, S=2K, 16/2 heads on 108 SMs
    # (one CTA resident per SM). Without splitting, 128 CTAs leave the second
    # wave nearly empty; 4-16 splits pack the waves and the model time drops.
    ns = fd.fd_plan_splits(64, 16, 2, 128, fd.FD_F16, [2048] * 64, 108, 0)
    assert 4 <= ns <= 16
    wgs = 128 * ns
    passes = math.ceil(wgs / 108)
    assert wgs / (passes * 108) > 128 / (2 * 108)


def test_planner_respects_max_splits():
    assert plan(1, 32, 8, 128, [131072], max_splits=4) <= 4


def test_planner_argument_errors():
    with pytest.raises(fd.FdError):
        plan(1, 30, 8, 128, [100])           # heads not a multiple of kv_heads
    with pytest.raises(fd.FdError) as e:
        plan(1, 32, 8, 100, [100])           # unsupported head dim
    assert e.value.status == 2
    with pytest.raises(fd.FdError):
        plan(0, 32, 8, 128, [])


# ---------------------------------------------------- argument rejection --
def _attn(lib, **kw):
    base = dict(q=16, k=16, v=16, cu=16, B=1, H=8, Hkv=1, D=128, ns=2, scale=0.1, out=16,
                ws=16, stream=None, dt=fd.FD_F16, lay=None)
    base.update(kw)
    return lib.fd_decode_attention(base["q"], base["k"], base["v"], base["cu"], base["B"],
                                   base["H"], base["Hkv"], base["D"], base["ns"],
                                   base["scale"], base["out"], base["ws"], base["stream"],
                                   base["dt"], base["lay"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(cu=None), 1), (dict(out=None), 1),
    (dict(ws=None), 1), (dict(B=0), 1), (dict(H=0), 1), (dict(H=9, Hkv=2), 1),
    (dict(ns=0), 1), (dict(ns=fd.FD_MAX_SPLITS + 1), 1), (dict(scale=float("inf")), 1),
    (dict(scale=float("nan")), 1), (dict(q=8), 1), (dict(D=96), 2), (dict(D=256), 2),
    (dict(dt=7), 2), (dict(H=65, Hkv=1), 2),
])
def test_decode_attention_rejects_before_launch(kw, status):
    assert _attn(_lib(), **kw) == status


def test_layout_checks():
    lib = _lib()
    bad = [fd.FdKvLayout(0, 128, 64, 0),      # token stride < dim
           fd.FdKvLayout(-1, 128, 128, 0),    # negative stride
           fd.FdKvLayout(0, 100, 128, 128),   # head stride not 16-byte aligned (fp16)
           fd.FdKvLayout(0, 128, 1 << 23, 0)]  # tile offsets would not fit 32 bits
    for lay in bad:
        assert _attn(lib, lay=ctypes.byref(lay)) == 1


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(cu=None), 1), (dict(out=None), 1), (dict(ws=None), 1),
    (dict(B=0), 1), (dict(H=9, Hkv=2), 1), (dict(ns=0), 1), (dict(scale=float("nan")), 1),
    (dict(D=96), 2), (dict(dt=7), 2),
])
def test_unnorm_attention_rejects_before_launch(kw, status):
    lib = _lib()
    base = dict(q=16, k=16, v=16, cu=16, B=1, H=8, Hkv=1, D=128, ns=2, scale=0.1, out=16,
                ws=16, stream=None, dt=fd.FD_F16, lay=None)
    base.update(kw)
    assert lib.fd_decode_attention_unnorm(
        base["q"], base["k"], base["v"], base["cu"], base["B"], base["H"], base["Hkv"],
        base["D"], base["ns"], base["scale"], base["out"], base["ws"], base["stream"],
        base["dt"], base["lay"]) == status
    assert lib.fd_decode_split_unnorm(16, 16, 16, 16, 1, 8, 1, 128, 2, 0.1, None, None, 1,
                                      None) == 1
    assert lib.fd_decode_combine_unnorm(None, 1, 8, 128, 2, 16, None, 1) == 1
    assert lib.fd_decode_combine_unnorm(16, 1, 8, 64 + 32, 2, 16, None, 1) == 2


def test_noalloc_rejects_before_launch():
    """fd_decode_attention_noalloc checks its arguments, then that the
    partials fit the static scratch, before touching any device."""
    lib = _lib()
    args = [16, 16, 16, 16]
    # 1 x 64 heads x 1100 splits x (128 + 1) floats > 16 MiB
    assert fd.fd_workspace_bytes(1, 64, 1100, 128) > fd.FD_NOALLOC_SCRATCH_BYTES
    assert lib.fd_decode_attention_noalloc(*args, 1, 64, 64, 128, 1100, 0.1, 16, None,
                                           fd.FD_F16, None) == 5
    assert "static scratch" in fd.fd_last_error()
    assert lib.fd_decode_attention_noalloc(*args, 1, 64, 64, 96, 2, 0.1, 16, None,
                                           fd.FD_F16, None) == 2
    assert lib.fd_decode_attention_noalloc(*args, 1, 64, 63, 128, 2, 0.1, 16, None,
                                           fd.FD_F16, None) == 1
    assert lib.fd_decode_attention_noalloc(None, 16, 16, 16, 1, 8, 1, 128, 1, 0.1, 16, None,
                                           fd.FD_F16, None) == 1
    assert lib.fd_decode_attention_noalloc(*args, 1, 8, 1, 128, 2, float("nan"), 16, None,
                                           fd.FD_F16, None) == 1
    assert "scratch" in fd.fd_status_string(5)


def test_split_and_combine_reject_before_launch():
    lib = _lib()
    assert lib.fd_decode_split(16, 16, 16, 16, 1, 8, 1, 128, 2, 0.1, None, None, 1, None) == 1
    assert lib.fd_decode_combine(None, 1, 8, 128, 2, 16, None, 1) == 1
    assert lib.fd_decode_combine(16, 1, 8, 128, 2, None, None, 1) == 1
    assert lib.fd_decode_combine(16, 1, 8, 96, 2, 16, None, 1) == 2
    assert lib.fd_decode_combine(16, 0, 8, 128, 2, 16, None, 1) == 1


def test_kernel_path_setting():
    prev = fd.fd_set_kernel_path(fd.FD_PATH_VALU)
    assert fd.fd_set_kernel_path(fd.FD_PATH_MFMA) == fd.FD_PATH_VALU
    assert fd.fd_set_kernel_path(fd.FD_PATH_UNPACKED) == fd.FD_PATH_MFMA
    assert fd.fd_set_kernel_path(prev) == fd.FD_PATH_UNPACKED
    assert _lib().fd_set_kernel_path(7) == -1
    with pytest.raises(ValueError):
        fd.fd_set_kernel_path(9)


def test_kernel_path_setting_is_per_thread():
    """Each thread steers only its own calls: a setting made on one thread is
    not seen by another, and a new thread starts at FD_PATH_AUTO."""
    import threading
    seen = {}
    gate = threading.Barrier(2)

    def worker(name, path):
        first = fd.fd_set_kernel_path(path)
        gate.wait()                       # both threads have set their path
        seen[name] = (first, fd.fd_set_kernel_path(first))

    main_prev = fd.fd_set_kernel_path(fd.FD_PATH_UNPACKED)
    try:
        ts = [threading.Thread(target=worker, args=("a", fd.FD_PATH_VALU)),
              threading.Thread(target=worker, args=("b", fd.FD_PATH_MFMA))]
        for t in ts:
            t.start()
        for t in ts:
            t.join()
    finally:
        assert fd.fd_set_kernel_path(main_prev) == fd.FD_PATH_UNPACKED
    assert seen == {"a": (fd.FD_PATH_AUTO, fd.FD_PATH_VALU),
                    "b": (fd.FD_PATH_AUTO, fd.FD_PATH_MFMA)}


# ------------------------------------------- binding argument marshalling --
def _cpu_inputs(B=2, H=8, Hkv=2, D=64, T=40):
    import torch
    q = torch.zeros(B, H, D, dtype=torch.float16)
    k = torch.zeros(T, Hkv, D, dtype=torch.float16)
    v = torch.zeros(T, Hkv, D, dtype=torch.float16)
    cu = torch.tensor([0, 10, T], dtype=torch.int32)
    return q, k, v, cu


def test_binding_refuses_mismatched_tensors_before_any_call():
    """The C ABI applies one stride set to K and V and reads one device: the
    binding refuses inputs that disagree before calling into the library."""
    import torch
    q, k, v, cu = _cpu_inputs()
    cases = [
        dict(v=torch.zeros(40, 2, 64, dtype=torch.float16).transpose(0, 1).contiguous()
             .transpose(0, 1)),                                     # other strides
        dict(v=torch.zeros(41, 2, 64, dtype=torch.float16)),        # other shape
        dict(k=k.float(), v=v.float()),                             # dtype differs from q
        dict(k=torch.zeros(40, 2, 32, dtype=torch.float16),
             v=torch.zeros(40, 2, 32, dtype=torch.float16)),        # head dim differs
        dict(cu=cu.long()),                                         # not int32
        dict(cu=torch.tensor([0, 40], dtype=torch.int32)),          # not batch + 1 entries
        dict(q=q.transpose(0, 1)),                                  # q not contiguous
    ]
    for c in cases:
        a = dict(q=q, k=k, v=v, cu=cu)
        a.update(c)
        with pytest.raises((ValueError, TypeError)):
            fd.fd_decode_attention(a["q"], a["k"], a["v"], a["cu"], 2)
        with pytest.raises((ValueError, TypeError)):
            fd.fd_decode_split(a["q"], a["k"], a["v"], a["cu"], 2)
    with pytest.raises(ValueError):
        fd.fd_decode_attention(q, k, v, cu, 2, out=torch.zeros(2, 8, 32, dtype=torch.float16))
    with pytest.raises(ValueError):
        fd.fd_decode_attention(q, k, v, cu, 2, layout="hbsd")


def test_binding_refuses_a_short_workspace_or_wrong_out_in_combine():
    import torch
    out = torch.zeros(2, 8, 64, dtype=torch.float16)
    need = fd.fd_workspace_bytes(2, 8, 3, 64)
    with pytest.raises(ValueError):
        fd.fd_decode_combine(torch.zeros(need - 1, dtype=torch.uint8), 2, 8, 64, 3, out)
    with pytest.raises(ValueError):
        fd.fd_decode_combine(torch.zeros(need, dtype=torch.uint8), 2, 8, 128, 3, out)


def test_kv_layout_strides():
    """Element strides handed to the C ABI for each layout name; row
    (b, t, j) starts at b*batch + cu[b]*cu + t*token + j*head."""
    import torch
    packed = torch.zeros(100, 4, 64)
    lay = fd.kv_layout(packed, "packed")
    assert (lay.batch_stride, lay.head_stride, lay.token_stride, lay.cu_stride) == (0, 64, 256, 256)
    bhsd = torch.zeros(3, 4, 50, 64)
    lay = fd.kv_layout(bhsd, "bhsd")
    assert (lay.batch_stride, lay.head_stride, lay.token_stride, lay.cu_stride) == (
        4 * 50 * 64, 50 * 64, 64, 0)
    bshd = torch.zeros(3, 50, 4, 64)
    lay = fd.kv_layout(bshd, "bshd")
    assert (lay.batch_stride, lay.head_stride, lay.token_stride, lay.cu_stride) == (
        50 * 4 * 64, 64, 4 * 64, 0)
    view = torch.zeros(3, 4, 80, 64)[:, :, :50]          # a cache with spare capacity
    lay = fd.kv_layout(view, "bhsd")
    assert (lay.batch_stride, lay.head_stride, lay.token_stride) == (4 * 80 * 64, 80 * 64, 64)
    with pytest.raises(ValueError):
        fd.kv_layout(torch.zeros(3, 4, 64, 50).transpose(2, 3), "bhsd")


def _model(B, H, Hkv, L, ns, cus=256, D=128, dtype=fd.FD_F16):
    return fd.fd_plan_time_us(B, H, Hkv, D, dtype, L if isinstance(L, list) else [L] * B, ns,
                              num_cus=cus)


@pytest.mark.parametrize("B,H,Hkv,L", [(1, 16, 2, 65536), (8, 16, 2, 8192), (64, 16, 2, 2048),
                                       (16, 32, 8, 131072), (1, 32, 8, 8192), (3, 28, 4, 40000)])
def test_planner_takes_the_least_modelled_time(B, H, Hkv, L):
    ns = plan(B, H, Hkv, 128, [L] * B)
    cap = min(math.ceil(L / 256), L)
    times = {n: _model(B, H, Hkv, L, n) for n in range(1, cap + 1)}
    assert times[ns] == min(times.values())
    assert all(times[n] > times[ns] for n in range(1, ns))   # ties go to fewer splits


def test_time_model_shows_demo4_wave_quantisation():
    # 04_flash_decoding.py, demo 4: too few splits leave compute units idle
    # (time falls as splits are added until one round fills the device),
    # beyond that more splits only add rounds and combine work
    t = [_model(8, 16, 2, 8192, n) for n in (1, 2, 4, 8, 16, 32, 64, 128)]
    assert t[0] > t[1] > t[2] > t[3] > t[4]        # 16 .. 256 workgroups
    assert t[4] == min(t) and t[7] > t[5] > t[4]
    # single launch for one split: no combine term; two splits add it
    one, two = _model(64, 16, 2, 2048, 1), _model(64, 16, 2, 2048, 2)
    assert one > two   # 128 workgroups leave half the device idle
    # bytes scale the time: twice the keys, about twice the streaming part
    assert _model(16, 32, 8, 65536, 2) > 1.9 * _model(16, 32, 8, 32768, 2) - 10


def test_time_model_argument_errors():
    with pytest.raises(ValueError):
        _model(1, 32, 8, 1000, 0)
    with pytest.raises(ValueError):
        fd.fd_plan_time_us(1, 30, 8, 128, fd.FD_F16, [100], 1, num_cus=256)


def test_planner_gives_the_steal_layout_under_the_steal_schedule():
    # under FD_SCHED_STEAL: shares per unit = CUs / units (at least 1), each
    # with 3 steal slots, where the matrix-core kernel runs (head dim 128,
    # group >= 2 or the matrix-core path forced) and every share of the
    # longest sequence has >= 1024 keys; otherwise the static plan
    static = {key: plan(*key[:4], [key[4]] * key[0], dtype=fd.FD_BF16)
              for key in ((16, 32, 8, 128, 1024), (16, 32, 8, 64, 131072),
                          (16, 32, 32, 128, 131072))}
    prev = fd.fd_set_schedule(fd.FD_SCHED_STEAL)
    try:
        assert plan(16, 32, 8, 128, [131072] * 16, dtype=fd.FD_BF16) == 8   # 128 units: 2 shares
        assert plan(1, 32, 8, 128, [131072], dtype=fd.FD_BF16) == 128       # 8 units: 32 shares
        assert plan(64, 32, 8, 128, [8192] * 64, dtype=fd.FD_BF16) == 4     # 512 units: 1 share
        assert plan(16, 32, 8, 128, [131072] * 16, cus=128, dtype=fd.FD_BF16) == 4
        # shares of 512 keys, head dim 64, MHA (VALU kernel): the static plan
        for key, ns in static.items():
            assert plan(*key[:4], [key[4]] * key[0], dtype=fd.FD_BF16) == ns
        prev_path = fd.fd_set_kernel_path(fd.FD_PATH_VALU)
        try:   # the VALU kernel has no steal schedule
            valu_steal = plan(16, 32, 8, 128, [131072] * 16, dtype=fd.FD_BF16)
        finally:
            fd.fd_set_kernel_path(prev_path)
    finally:
        fd.fd_set_schedule(prev)
    assert valu_steal == plan(16, 32, 8, 128, [131072] * 16, dtype=fd.FD_BF16) != 8


def test_plan_schedule_recommends_steal_for_long_even_shares():
    # near-uniform batches: the steal schedule where it measured faster on
    # MI355X: matrix-core kernel (head dim 128), lengths within 1.5x, shares
    # of >= 12 MB of K+V
    def ps(B, H, Hkv, D, lens, dtype=fd.FD_BF16, cus=256):
        return fd.fd_plan_schedule(B, H, Hkv, D, dtype, lens, cus, 0)
    steal, static = fd.FD_SCHED_STEAL, fd.FD_SCHED_STATIC
    assert ps(16, 32, 8, 128, [131072] * 16) == (steal, 8)      # 32 MB shares
    assert ps(16, 32, 8, 128, [65536] * 16) == (steal, 8)       # 16.8 MB
    assert ps(2, 32, 8, 128, [1 << 20] * 2) == (steal, 64)      # 16 units: 16 shares each
    assert ps(16, 32, 8, 128, [131072] * 8 + [98304] * 8) == (steal, 8)   # within 1.5x
    # shorter shares, other kernels: the static plan
    for args, kw in (((16, 32, 8, 128, [32768] * 16), {}),            # 8.4 MB shares
                     ((1, 32, 8, 128, [131072]), {}),                 # 2 MB shares
                     ((16, 32, 8, 64, [131072] * 16), {}),            # head dim 64
                     ((16, 32, 32, 128, [131072] * 16), {}),          # MHA: VALU kernel
                     ((32, 28, 4, 128, [32768] * 32), {"dtype": fd.FD_F16})):
        sched, ns = ps(*args, **kw)
        assert sched == static, args
        assert ns == fd.fd_plan_splits(*args[:4], kw.get("dtype", fd.FD_BF16), args[4], 256, 0)
    prev = fd.fd_set_kernel_path(fd.FD_PATH_VALU)
    try:
        assert ps(16, 32, 8, 128, [131072] * 16)[0] == static
    finally:
        fd.fd_set_kernel_path(prev)
    with pytest.raises(fd.FdError):
        ps(2, 32, 8, 128, [5, 0])


def test_plan_schedule_recommends_the_queue_for_ragged_batches():
    # longest >= 1.5x shortest: the queue schedule at ~4 segments per CU,
    # round(4 * cus / units) splits, capped by the shortest sequence and
    # 256 keys per split of the longest, where the launch fills the device
    def ps(B, H, Hkv, D, lens, dtype=fd.FD_F16, cus=256):
        return fd.fd_plan_schedule(B, H, Hkv, D, dtype, lens, cus, 0)
    queue, static = fd.FD_SCHED_QUEUE, fd.FD_SCHED_STATIC
    rng = np.random.default_rng(5)
    varlen = [int(x) for x in rng.integers(64, 32769, size=32)]
    assert ps(32, 28, 4, 128, varlen) == (queue, 8)                         # 128 units
    assert ps(16, 32, 8, 128, [131072] * 8 + [32768] * 8, fd.FD_BF16) == (queue, 8)
    assert ps(4, 32, 8, 128, [8192, 65536, 20000, 40000], fd.FD_BF16) == (queue, 32)
    assert ps(32, 28, 4, 64, varlen) == (queue, 8)        # any head dim and kernel
    assert ps(32, 28, 4, 128, varlen, cus=80) == (queue, 3)   # round(320 / 128)
    # capped by the shortest sequence
    assert ps(32, 28, 4, 128, [5] + [30000] * 31) == (queue, 5)
    # a ragged launch that cannot fill the device: not the queue
    sched, ns = ps(2, 8, 1, 128, [3000, 1000])
    assert sched != queue
