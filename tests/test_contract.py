"""Host contract of the C ABI, exercised without a GPU through the host-only
twin mnb_prepare_host and through argument checks that fail before any HIP
call.

Contract sources: "Qwen3 Missing-Kernel Implementation Plan", section "PR
sequence", step K01 (FP32/UINT8/FP32 contract, bits=4, block_size=32,
accuracy_level=4, implicit zero points, padding, explicit rejection of
unsupported variants); onnxruntime PR "INT3 QMoE CUDA correctness baseline and
Qwen experimental results", embedded P0/P1 body, sections "P0" (checked size
arithmetic, canonical padding), "P1" (INT3 profile, finite nonnegative FP16
scales, block-aligned K) and "Latest Review Fixes" (N = 127 accepted).
"""
import ctypes

import numpy as np
import pytest

import block_quantized_weight_03_amd as mnb
import synth

OK, INVALID, UNSUP, OVERFLOW, CONTENT, SMALL, DEVICE, STALE = 0, -1, -2, -3, -4, -5, -6, -7


def status_of(fn, *args):
    try:
        fn(*args)
        return OK
    except mnb.MnbError as e:
        return e.status


def size_status(desc):
    return status_of(mnb.mnb_prepacked_size, desc)


def dense_inputs(N, K, bs=32, zp=False, seed=1):
    nb = -(-K // bs)
    B = synth.int4_blocked_weights(seed, N, K, bs)
    s = synth.scales_f32(seed + 1, (N, nb))
    Z = synth.int4_zero_points(seed + 2, N, nb) if zp else None
    return B, s, Z


def host_prepare(desc, B, s, Z):
    dst = np.zeros(mnb.mnb_prepacked_size(desc) + 512, np.uint8)
    off = (-dst.ctypes.data) % 256
    view = dst[off:off + mnb.mnb_prepacked_size(desc)]
    plan = mnb.mnb_prepare_host(desc, B, s, Z, view)
    return plan, view, dst


def test_descriptor_rejections():
    good = mnb.dense_desc(64, 16)
    assert size_status(good) == OK

    def with_(**kw):
        d = mnb.dense_desc(64, 16)
        for k, v in kw.items():
            setattr(d, k, v)
        return d

    assert size_status(with_(abi_version=2)) == INVALID
    for bits in (1, 2, 5, 8):
        assert size_status(with_(bits=bits)) == UNSUP
    for bits in (0, 9, -1):
        assert size_status(with_(bits=bits)) == INVALID
    for bs in (16, 256, 48):
        assert size_status(with_(block_size=bs)) == UNSUP
    assert size_status(with_(block_size=0)) == INVALID
    for lvl in (-1, 5):
        assert size_status(with_(accuracy_level=lvl)) == INVALID
    for lvl in range(5):
        assert size_status(with_(accuracy_level=lvl)) == OK
    assert size_status(with_(K=0)) == INVALID
    assert size_status(with_(N=0)) == INVALID
    assert size_status(with_(N=-3)) == INVALID
    assert size_status(with_(num_experts=0)) == INVALID
    assert size_status(with_(scale_dtype=mnb.MNB_DTYPE_F16)) == UNSUP
    assert size_status(with_(row_layout=mnb.MNB_ROWS_ROW_LOCAL)) == UNSUP
    assert size_status(with_(num_experts=2)) == UNSUP
    assert size_status(with_(has_zero_points=2)) == INVALID
    assert size_status(with_(scale_dtype=7)) == INVALID
    # INT3 QMoE profile
    q = mnb.qmoe_proj_desc(2048, 1536, 128, 64)
    assert size_status(q) == OK
    size = mnb.mnb_prepacked_size(q)
    q.has_zero_points = 1  # explicit zero points: validated, then implied
    assert size_status(q) == OK and mnb.mnb_prepacked_size(q) == size
    assert size_status(mnb.qmoe_proj_desc(100, 8, 2, 64)) == UNSUP  # K not block aligned
    q = mnb.qmoe_proj_desc(128, 8, 2, 64)
    q.scale_dtype = mnb.MNB_DTYPE_F32
    assert size_status(q) == UNSUP
    # INT4 QMoE projections (width pairs (3,4), (4,3), (4,4)): same profile
    assert size_status(mnb.qmoe_proj_desc(2048, 1536, 128, 64, bits=4)) == OK
    assert size_status(mnb.qmoe_proj_desc(96, 8, 2, 64, bits=4)) == UNSUP  # K not block aligned
    for bits in (2, 5, 8):
        assert size_status(mnb.qmoe_proj_desc(128, 8, 2, 64, bits=bits)) == UNSUP
    q = mnb.qmoe_proj_desc(128, 8, 2, 64, bits=4)
    q.row_layout = mnb.MNB_ROWS_BLOCKED
    assert size_status(q) == UNSUP


def test_size_overflow_is_detected():
    d = mnb.dense_desc(2 ** 40, 2 ** 40)
    assert size_status(d) == OVERFLOW
    d = mnb.dense_desc(2 ** 62, 8)
    assert size_status(d) == OVERFLOW
    q = mnb.qmoe_proj_desc(2 ** 61, 2 ** 10, 4, 64)
    assert size_status(q) == OVERFLOW


@pytest.mark.parametrize("K,N,bs,zp", [(2048, 2048, 32, False), (2050, 1024, 32, False),
                                       (2048, 151936, 32, True), (6144, 2048, 64, False),
                                       (33, 127, 128, True)])
def test_prepacked_size_never_inflates(K, N, bs, zp):
    nb = -(-K // bs)
    contract = N * nb * bs // 2 + N * nb * 4 + (N * ((nb + 1) // 2) if zp else 0)
    size = mnb.mnb_prepacked_size(mnb.dense_desc(K, N, bs, zp))
    assert contract <= size <= contract + 768


@pytest.mark.parametrize("K,N,bs,zp", [(64, 16, 32, False), (2050, 33, 32, True), (34, 5, 32, False),
                                       (200, 127, 64, True), (130, 3, 128, False)])
def test_dense_host_prepack_round_trip(orc, K, N, bs, zp):
    B, s, Z = dense_inputs(N, K, bs, zp, seed=K + N)
    desc = mnb.dense_desc(K, N, bs, zp)
    plan, _, _keep = host_prepare(desc, B, s, Z)
    assert plan.device == -1 and plan.layout_version >= 1
    codes, zeros, scales = mnb.mnb_debug_unpack_host(plan, 0, 0, N)
    ocodes, ozeros = orc.mnb_codes(B, Z, K, N, bs=bs)
    assert np.array_equal(codes, ocodes)
    assert np.array_equal(zeros, ozeros)
    assert np.array_equal(scales, s)
    # a sub-range of rows
    c2, _, _ = mnb.mnb_debug_unpack_host(plan, 0, 1, N - 1)
    assert np.array_equal(c2, ocodes[1:])


def test_pad_codes_do_not_change_the_prepared_codes(orc):
    K, N, bs = 2050, 4, 32
    Bz = synth.int4_blocked_weights(9, N, K, bs, pad="zero")
    Br = synth.int4_blocked_weights(9, N, K, bs, pad="random")
    s = synth.scales_f32(10, (N, 65))
    pz, vz, _a = host_prepare(mnb.dense_desc(K, N, bs), Bz, s, None)
    pr, vr, _b = host_prepare(mnb.dense_desc(K, N, bs), Br, s, None)
    assert not np.array_equal(Bz, Br)
    assert np.array_equal(vz, vr)  # pad nibbles are normalised by the prepack


def test_int3_host_prepack_round_trip_and_n127(orc):
    E, N, K, bs = 3, 127, 256, 64
    W = synth.int3_rows(4, E * N, K)
    s = synth.scales_f16(5, (E * N, K // bs))
    desc = mnb.qmoe_proj_desc(K, N, E, bs)
    plan, _, _keep = host_prepare(desc, W, s, None)
    for e in range(E):
        codes, zeros, sc = mnb.mnb_debug_unpack_host(plan, e, 0, N)
        ref = np.stack([orc.unpack_bits(W[e * N + r], K, 3) for r in range(N)])
        assert np.array_equal(codes, ref)
        assert (zeros == 4).all()
        assert np.array_equal(sc.view(np.uint16), s[e * N:(e + 1) * N].view(np.uint16))


@pytest.mark.parametrize("E,N,K,bs", [(3, 127, 256, 64), (2, 16, 128, 32), (1, 5, 384, 128),
                                      (2, 40, 96, 32)])
def test_int4_moe_host_prepack_round_trip(orc, E, N, K, bs):
    """4-bit row-local rows regrouped into the private groups read back as the
    oracle's codes (low nibble = even position), zero point 8, scales as given."""
    W = synth.packed_rows(E * N + K, E * N, K, 4)
    s = synth.scales_f16(5, (E * N, K // bs))
    desc = mnb.qmoe_proj_desc(K, N, E, bs, bits=4)
    assert mnb.mnb_prepacked_size(desc) <= W.nbytes + s.nbytes + 768
    plan, _, _keep = host_prepare(desc, W, s, None)
    for e in range(E):
        codes, zeros, sc = mnb.mnb_debug_unpack_host(plan, e, 0, N)
        ref = np.stack([orc.unpack_bits(W[e * N + r], K, 4) for r in range(N)])
        assert np.array_equal(codes, ref)
        assert (zeros == 8).all()
        assert np.array_equal(sc.view(np.uint16), s[e * N:(e + 1) * N].view(np.uint16))


@pytest.mark.parametrize("bits", [3, 4])
def test_moe_host_prepack_threaded_stack(bits):
    """A stack above 8 MB is repacked tile by tile on several host threads;
    whole experts (first, middle, last; N = 1000 leaves an 8-row last tile)
    read back as numpy's LSB-first unpack of the contract rows."""
    E, N, K, bs = 16, 1000, 2048, 64
    W = synth.packed_rows(900 + bits, E * N, K, bits)
    assert W.nbytes > (8 << 20)
    s = synth.scales_f16(901, (E * N, K // bs))
    plan, _, _keep = host_prepare(mnb.qmoe_proj_desc(K, N, E, bs, bits=bits), W, s, None)
    weights = (1 << np.arange(bits)).astype(np.int64)
    for e in (0, 7, 15):
        codes, _, _ = mnb.mnb_debug_unpack_host(plan, e, 0, N, want_scales=False)
        rows = W[e * N:(e + 1) * N]
        ref = np.unpackbits(rows, axis=1, bitorder="little")[:, :K * bits].reshape(N, K, bits) @ weights
        assert np.array_equal(codes, ref)


@pytest.mark.parametrize("bits", [3, 4])
@pytest.mark.parametrize("bad", [np.inf, -np.inf, np.nan, -0.5, -65504.0])
def test_moe_scale_content_rejected(bad, bits):
    E, N, K, bs = 2, 4, 128, 64
    W = synth.packed_rows(4, E * N, K, bits)
    s = synth.scales_f16(5, (E * N, K // bs))
    s[3, 1] = np.float16(bad)
    desc = mnb.qmoe_proj_desc(K, N, E, bs, bits=bits)
    with pytest.raises(mnb.MnbError) as ei:
        host_prepare(desc, W, s, None)
    assert ei.value.status == CONTENT


def test_int3_negative_zero_and_zero_scales_accepted():
    E, N, K, bs = 1, 2, 64, 64
    W = synth.int3_rows(4, E * N, K)
    s = np.array([[-0.0], [0.0]], np.float16)
    host_prepare(mnb.qmoe_proj_desc(K, N, E, bs), W, s, None)


def test_prepare_argument_errors():
    K, N = 64, 8
    B, s, Z = dense_inputs(N, K)
    desc = mnb.dense_desc(K, N)
    need = mnb.mnb_prepacked_size(desc)
    buf = np.zeros(need + 512, np.uint8)
    off = (-buf.ctypes.data) % 256
    ok_view = buf[off:off + need]
    assert status_of(mnb.mnb_prepare_host, desc, B, s, None, ok_view) == OK
    assert status_of(mnb.mnb_prepare_host, desc, B, s, None, buf[off:off + need - 1]) == SMALL
    assert status_of(mnb.mnb_prepare_host, desc, B, s, None, buf[off + 1:off + 1 + need]) == INVALID
    zdesc = mnb.dense_desc(K, N, has_zero_points=True)
    zneed = mnb.mnb_prepacked_size(zdesc)
    assert status_of(mnb.mnb_prepare_host, zdesc, B, s, None, buf[off:off + zneed]) == INVALID
    lib = mnb.lib()
    plan = mnb.mnb_plan()
    assert lib.mnb_prepare_host(ctypes.byref(desc), None, s.ctypes.data, None,
                                ok_view.ctypes.data, need, ctypes.byref(plan)) == INVALID
    assert lib.mnb_prepare_host(ctypes.byref(desc), B.ctypes.data, s.ctypes.data, None,
                                ok_view.ctypes.data, need, None) == INVALID
    # a failed prepare leaves a zeroed plan
    plan.magic = 123
    assert lib.mnb_prepare_host(ctypes.byref(desc), B.ctypes.data, s.ctypes.data, None,
                                ok_view.ctypes.data, 1, ctypes.byref(plan)) == SMALL
    assert plan.magic == 0


def test_stale_and_mismatched_plans_rejected_before_any_launch():
    K, N = 64, 8
    B, s, _ = dense_inputs(N, K)
    plan, _, _keep = host_prepare(mnb.dense_desc(K, N), B, s, None)
    assert mnb.mnb_gemv_workspace_size(plan) == 0  # K <= 8192: one fused launch
    Kl = 8192 + 32
    Bl, sl, _ = dense_inputs(N, Kl)
    plan_l, _, _keep_l = host_prepare(mnb.dense_desc(Kl, N), Bl, sl, None)
    assert mnb.mnb_gemv_workspace_size(plan_l) > 0  # longer K: digit pre-pass in ws
    lib = mnb.lib()
    out = ctypes.c_uint64()
    for field, val in (("magic", 1), ("layout_version", 999), ("codes_bytes", 7)):
        bad = mnb.mnb_plan.from_buffer_copy(plan)
        setattr(bad, field, val)
        assert lib.mnb_gemv_workspace_size(ctypes.byref(bad), ctypes.byref(out)) == STALE
        assert lib.mnb_gemv(ctypes.byref(bad), 1, 1, 1, 1 << 20, None) == STALE
    bad = mnb.mnb_plan.from_buffer_copy(plan)
    bad.desc.K = 65
    assert lib.mnb_gemv_workspace_size(ctypes.byref(bad), ctypes.byref(out)) == STALE
    # argument errors are found before any HIP call
    assert lib.mnb_gemv(ctypes.byref(plan), None, 1, 1, 1 << 20, None) == INVALID
    assert lib.mnb_gemv(ctypes.byref(plan_l), 1, 1, None, 0, None) == SMALL
    assert lib.mnb_gemv(ctypes.byref(plan_l), 1, 1, 256, 1, None) == SMALL
    assert lib.mnb_gemm(ctypes.byref(plan), -1, 1, 1, None, 0, None) == INVALID
    assert lib.mnb_gemm(ctypes.byref(plan), 0, None, None, None, 0, None) == OK  # M = 0: no-op
    assert lib.mnb_gemm(ctypes.byref(plan), 2 ** 62, 1, 1, None, 0, None) == OVERFLOW
    assert lib.mnb_debug_unpack_host(ctypes.byref(plan), 1, 0, 1, None, None, None) == INVALID
    assert lib.mnb_debug_unpack_host(ctypes.byref(plan), 0, 5, 4, None, None, None) == INVALID


def test_qmoe_descriptor_and_shape_checks():
    E, H, I, bs = 4, 128, 64, 64
    W1 = synth.int3_rows(1, E * 2 * I, H)
    s1 = synth.scales_f16(2, (E * 2 * I, H // bs))
    W2 = synth.int3_rows(3, E * H, I)
    s2 = synth.scales_f16(4, (E * H, I // bs))
    p1, _, _k1 = host_prepare(mnb.qmoe_proj_desc(H, 2 * I, E, bs), W1, s1, None)
    p2, _, _k2 = host_prepare(mnb.qmoe_proj_desc(I, H, E, bs), W2, s2, None)
    q = mnb.make_qmoe_desc(2)
    assert mnb.qmoe_workspace_size(p1, p2, q, 16) >= 0
    assert status_of(mnb.qmoe_workspace_size, p2, p1, q, 16) == INVALID  # swapped projections
    assert status_of(mnb.qmoe_workspace_size, p1, p2, q, -1) == INVALID
    for field, val, want in (("top_k", 0, INVALID), ("top_k", E + 1, INVALID),
                             ("normalize_routing_weights", 0, UNSUP), ("activation", 0, UNSUP),
                             ("gate_up", 0, UNSUP), ("weights_prepacked", 1, UNSUP),
                             ("quant_type", 1, UNSUP), ("abi_version", 0, INVALID)):
        bad = mnb.make_qmoe_desc(2)
        setattr(bad, field, val)
        assert status_of(mnb.qmoe_workspace_size, p1, p2, bad, 16) == want, field
    lib = mnb.lib()
    assert lib.qmoe_forward(ctypes.byref(p1), ctypes.byref(p2), ctypes.byref(q), 0, None, None,
                            None, None, 0, None) == OK  # T = 0: no-op
    # mixed widths: an INT4 FC2 next to the INT3 FC1 is a valid layer
    W2b = synth.packed_rows(5, E * H, I, 4)
    p2b, _, _k4 = host_prepare(mnb.qmoe_proj_desc(I, H, E, bs, bits=4), W2b, s2, None)
    assert mnb.qmoe_workspace_size(p1, p2b, q, 16) == mnb.qmoe_workspace_size(p1, p2, q, 16)
    # a dense plan is not a QMoE projection
    B, s, _ = dense_inputs(8, 64)
    pd, _, _k3 = host_prepare(mnb.dense_desc(64, 8), B, s, None)
    assert status_of(mnb.qmoe_workspace_size, pd, p2, q, 4) == UNSUP
    assert lib.mnb_gemv(ctypes.byref(p1), 1, 1, 256, 1 << 20, None) == UNSUP


def test_qmoe_kernel_limits_are_unsupported():
    """More than 1024 experts or top_k above 16 are valid requests that the
    built kernels do not run: both qmoe_workspace_size and qmoe_forward
    report UNSUPPORTED before any device call."""
    H, I, bs = 32, 32, 32

    def plans(E):
        W1 = synth.int3_rows(11, E * 2 * I, H)
        s1 = synth.scales_f16(12, (E * 2 * I, H // bs))
        W2 = synth.int3_rows(13, E * H, I)
        s2 = synth.scales_f16(14, (E * H, I // bs))
        p1, _, k1 = host_prepare(mnb.qmoe_proj_desc(H, 2 * I, E, bs), W1, s1, None)
        p2, _, k2 = host_prepare(mnb.qmoe_proj_desc(I, H, E, bs), W2, s2, None)
        return p1, p2, (k1, k2)

    lib = mnb.lib()
    for E, k, want in ((1024, 16, OK), (1025, 8, UNSUP), (32, 17, UNSUP), (32, 16, OK)):
        p1, p2, keep = plans(E)
        q = mnb.make_qmoe_desc(k)
        got = status_of(mnb.qmoe_workspace_size, p1, p2, q, 4) if want else 0
        if want:
            assert got == want, (E, k)
        else:
            assert mnb.qmoe_workspace_size(p1, p2, q, 4) > 0
        if want:
            assert lib.qmoe_forward(ctypes.byref(p1), ctypes.byref(p2), ctypes.byref(q), 4, 16, 16,
                                    16, 256, 1 << 30, None) == want, (E, k)


def test_gemv_multi_argument_checks_before_any_device_call():
    """mnb_gemv_multi rejects a plan count outside [1, 4], a missing output and
    plans of different K before it touches a device (host plans suffice)."""
    p1, v1, d1 = host_prepare(mnb.dense_desc(64, 16), *dense_inputs(16, 64))
    p2, v2, d2 = host_prepare(mnb.dense_desc(96, 16), *dense_inputs(16, 96, seed=5))
    y = np.zeros(16, np.float32)
    a = np.zeros(96, np.float32)
    assert status_of(mnb.mnb_gemv_multi, [], a, [], None, 0, 0) == INVALID
    assert status_of(mnb.mnb_gemv_multi, [p1] * 5, a, [y] * 5, None, 0, 0) == INVALID
    assert status_of(mnb.mnb_gemv_multi, [p1, p1], a, [y, None], None, 0, 0) == INVALID
    assert status_of(mnb.mnb_gemv_multi, [p1, p2], a, [y, y], None, 0, 0) == INVALID
    assert status_of(mnb.mnb_gemv_multi, [p1, p2], None, [y, y], None, 0, 0) == INVALID


def test_quantizer_argument_checks_before_any_device_call():
    """Every check of mnb_quantize_int3_rtn runs on the host before a launch."""
    lib = mnb.lib()
    f = lib.mnb_quantize_int3_rtn
    F16, BF16 = mnb.MNB_DTYPE_F16, mnb.MNB_DTYPE_BF16
    assert f(None, 0, 64, 32, F16, None, None, None, None) == OK  # rows = 0: no-op
    assert f(None, 0, 64, 32, BF16, None, None, None, None) == OK
    assert f(16, 4, 64, 48, F16, 16, 16, 16, None) == UNSUP      # block size
    assert f(16, 4, 96, 64, BF16, 16, 16, 16, None) == UNSUP     # K not block aligned
    assert f(16, 4, 64, 32, mnb.MNB_DTYPE_F32, 16, 16, 16, None) == UNSUP  # fp32 scales
    assert f(16, 4, 64, 32, 3, 16, 16, 16, None) == INVALID      # unknown scale type
    assert f(16, 4, 64, 32, -1, 16, 16, 16, None) == INVALID
    assert f(16, 4, 64, 0, F16, 16, 16, 16, None) == INVALID
    assert f(16, -1, 64, 32, F16, 16, 16, 16, None) == INVALID
    assert f(16, 4, 0, 32, F16, 16, 16, 16, None) == INVALID
    assert f(None, 4, 64, 32, F16, 16, 16, 16, None) == INVALID  # null weights
    assert f(16, 4, 64, 32, F16, 16, None, 16, None) == INVALID  # null scales
    assert f(8, 4, 64, 32, F16, 16, 16, 16, None) == INVALID     # weights not 16-byte aligned
    assert f(16, 4, 64, 32, F16, 18, 16, 16, None) == INVALID    # codes not 4-byte aligned
    assert f(16, 4, 64, 32, BF16, 16, 17, 16, None) == INVALID   # scales not 2-byte aligned
    assert f(16, 2 ** 40, 2 ** 30, 32, F16, 16, 16, 16, None) == OVERFLOW


@pytest.mark.parametrize("bits,K,bs", [(3, 128, 64), (4, 128, 32), (3, 320, 32), (4, 384, 128)])
def test_moe_explicit_zero_points_must_equal_the_implicit_value(orc, bits, K, bs):
    """Packed per-row block zero points of a QMoE projection are accepted only
    when every one is 2^(bits-1) with canonical padding; the prepared bytes
    are then those of the implicit-zero-point plan."""
    E, N = 2, 24
    nb = K // bs
    W = synth.packed_rows(bits + K, E * N, K, bits)
    s = synth.scales_f16(6, (E * N, nb))
    zrow = orc.pack_bits(np.full(nb, 1 << (bits - 1), np.uint8), bits)
    Z = np.tile(zrow, (E * N, 1))
    d0 = mnb.qmoe_proj_desc(K, N, E, bs, bits=bits)
    dz = mnb.qmoe_proj_desc(K, N, E, bs, bits=bits)
    dz.has_zero_points = 1
    _, v0, _k0 = host_prepare(d0, W, s, None)
    _, vz, _kz = host_prepare(dz, W, s, Z)
    assert np.array_equal(v0, vz)
    bad = Z.copy()
    bad[E * N - 1] = orc.pack_bits(np.array([1 << (bits - 1)] * (nb - 1) + [(1 << (bits - 1)) - 1],
                                            np.uint8), bits)
    with pytest.raises(mnb.MnbError) as e:
        host_prepare(dz, W, s, bad)
    assert e.value.status == CONTENT
    if (nb * bits) % 8:
        pad = Z.copy()
        pad[3, -1] |= np.uint8(0x80)  # a set pad bit after nb * bits
        with pytest.raises(mnb.MnbError) as e:
            host_prepare(dz, W, s, pad)
        assert e.value.status == CONTENT


@pytest.mark.parametrize("bad", [0x7F80, 0xFF80, 0x7FC0, 0xBF00, 0x8001])
def test_bf16_moe_scale_content_rejected(bad):
    """bfloat16 QMoE scales: finite and nonnegative (exponent 0xFF is Inf/NaN;
    a sign bit only on zero)."""
    E, N, K, bs = 2, 4, 128, 64
    W = synth.packed_rows(4, E * N, K, 3)
    s = synth.scales_bf16(5, (E * N, K // bs))
    desc = mnb.qmoe_proj_desc(K, N, E, bs, 3, mnb.MNB_DTYPE_BF16)
    ok = s.copy()
    ok[0, 0] = 0x8000  # -0 is accepted
    host_prepare(desc, W, ok, None)
    s[3, 1] = bad
    with pytest.raises(mnb.MnbError) as ei:
        host_prepare(desc, W, s, None)
    assert ei.value.status == CONTENT


def test_qmoe_layer_dtypes_must_match():
    E, H, I, bs = 4, 128, 64, 64
    p = {}
    keep = []
    for dt in (mnb.MNB_DTYPE_F16, mnb.MNB_DTYPE_BF16):
        W1 = synth.packed_rows(1, E * 2 * I, H, 3)
        W2 = synth.packed_rows(3, E * H, I, 3)
        s1 = synth.scales_bf16(2, (E * 2 * I, H // bs))  # any bits: valid in both formats
        s2 = synth.scales_bf16(4, (E * H, I // bs))
        p1, _, k1 = host_prepare(mnb.qmoe_proj_desc(H, 2 * I, E, bs, 3, dt), W1, s1, None)
        p2, _, k2 = host_prepare(mnb.qmoe_proj_desc(I, H, E, bs, 3, dt), W2, s2, None)
        p[dt] = (p1, p2)
        keep += [k1, k2]
    q = mnb.make_qmoe_desc(2)
    assert mnb.qmoe_workspace_size(*p[mnb.MNB_DTYPE_BF16], q, 8) == \
        mnb.qmoe_workspace_size(*p[mnb.MNB_DTYPE_F16], q, 8)
    assert status_of(mnb.qmoe_workspace_size, p[mnb.MNB_DTYPE_F16][0], p[mnb.MNB_DTYPE_BF16][1],
                     q, 8) == UNSUP


def test_biased_qmoe_pointer_checks_before_any_device_call():
    """qmoe_forward_biased rejects misaligned activations, outputs and biases
    before it touches a device (host plans suffice to reach those checks)."""
    E, H, I, bs = 4, 128, 64, 64
    W1 = synth.packed_rows(1, E * 2 * I, H, 4)
    W2 = synth.packed_rows(3, E * H, I, 3)
    s1 = synth.scales_f16(2, (E * 2 * I, H // bs))
    s2 = synth.scales_f16(4, (E * H, I // bs))
    p1, _, _k1 = host_prepare(mnb.qmoe_proj_desc(H, 2 * I, E, bs, 4), W1, s1, None)
    p2, _, _k2 = host_prepare(mnb.qmoe_proj_desc(I, H, E, bs, 3), W2, s2, None)
    q = mnb.make_qmoe_desc(2)
    lib = mnb.lib()
    f = lib.qmoe_forward_biased
    args = lambda x, b1, b2, out: (ctypes.byref(p1), ctypes.byref(p2), ctypes.byref(q), 8, x, 4096,
                                   b1, b2, out, 1 << 20, 1 << 30, None)
    assert f(*args(4096 + 8, None, None, 8192)) == INVALID   # x not 16-byte aligned
    assert f(*args(4096, None, None, 8192 + 4)) == INVALID   # out not 8-byte aligned
    assert f(*args(4096, 1001, None, 8192)) == INVALID       # FC1 bias not 2-byte aligned
    assert f(*args(4096, None, 3, 8192)) == INVALID          # FC2 bias not 2-byte aligned
    assert f(*args(None, None, None, 8192)) == INVALID       # no activations
    assert f(ctypes.byref(p1), ctypes.byref(p2), ctypes.byref(q), 0, None, None, None, None, None,
             None, 0, None) == OK                            # T = 0: no-op


def test_stream_read_argument_checks_before_any_device_call():
    lib = mnb.lib()
    P = ctypes.c_void_p * 2
    U = ctypes.c_uint64 * 2
    sink = ctypes.c_void_p(256)
    assert lib.mnb_debug_stream_read(P(256, 512), U(16, 32), 0, sink, None) == INVALID
    assert lib.mnb_debug_stream_read(P(256, 512), U(16, 32), 5, sink, None) == INVALID
    assert lib.mnb_debug_stream_read(P(256, 520), U(16, 32), 2, sink, None) == INVALID  # misaligned
    assert lib.mnb_debug_stream_read(P(256, 512), U(16, 33), 2, sink, None) == INVALID  # size
    assert lib.mnb_debug_stream_read(P(256, None), U(16, 32), 2, sink, None) == INVALID
    assert lib.mnb_debug_stream_read(P(256, 512), U(16, 32), 2, None, None) == INVALID
