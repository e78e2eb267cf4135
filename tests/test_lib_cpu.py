"""Host-side checks of libkvtc that need no GPU: the C ABI loads and exports
every declared symbol, artifacts interoperate byte for byte with the oracle's
format, sizes match, errors are reported, and the library's calibration
agrees with the oracle's (eigenvalues, group projectors, DP widths)."""
import os
import re
import zlib

import numpy as np
import pytest

import kv_cache_transform_amd as K
import oracle.kvtc_oracle as O
import pins
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _params_pair(w, max_bits=8):
    dt = O.DTYPE_F32 if w.dtype == "f32" else O.DTYPE_BF16
    op = O.Params(w.n_layers, w.kv_heads, w.head_dim, w.sink, w.window, w.group, max_bits,
                  w.bits_per_value, dt)
    kp = K.params(w.n_layers, w.kv_heads, w.head_dim, w.sink, w.window, w.group, max_bits,
                  w.bits_per_value, dt)
    return op, kp


def test_exports_every_declared_symbol():
    header = open(os.path.join(ROOT, "include", "kvtc.h")).read()
    declared = set(re.findall(r"\b(kvtc_[a-z_]+)\s*\(", header))
    L = K.lib()
    missing = [s for s in sorted(declared) if not hasattr(L, s)]
    assert not missing, missing
    assert len(declared) >= 20
    assert K.kvtc_version().startswith("kvtc")


def test_calibration_matches_oracle_tiny():
    w = synth.workload("tiny")
    op, kp = _params_pair(w)
    x = synth.gen_kv(w, 0, 0, 1, w.calib_tokens)
    c = K.Codec(kp)
    c.calibrate(0, 0, synth.storage(w, x), threads=4)
    so = O.calibrate(x, op, 0, 0)
    sl = O.parse_artifact(c.save()).slots[(0, 0)]
    _compare_slots(sl, so)


def _compare_slots(sl, so):
    assert np.array_equal(sl.mu32, so.mu32)
    lam_ok = so.lam > so.lam[0] * 1e-12
    assert np.allclose(sl.lam[lam_ok], so.lam[lam_ok], rtol=1e-6)
    if np.array_equal(sl.widths, so.widths):
        G = so.G
        for a, g in enumerate(so.active_groups):
            Vl = sl.V32[:, a * G:(a + 1) * G].astype(np.float64)
            Vo = so.V64[:, g * G:(g + 1) * G]
            assert np.abs(Vl @ Vl.T - Vo @ Vo.T).max() <= 1e-5
    else:  # a near-tie may flip: the objective must still agree
        obj = lambda wv: sum(so.D[g, b] for g, b in enumerate(wv))
        assert abs(obj(sl.widths) - obj(so.widths)) <= 1e-9 * obj(so.widths)


@pytest.mark.parametrize("kind", [0, 1])
def test_calibration_matches_oracle_llama8b_tensor(kind):
    w = synth.workload("llama31_8b")
    op, kp = _params_pair(w)
    x = synth.gen_kv(w, 3, kind, 1, w.calib_tokens)
    c = K.Codec(kp)
    c.calibrate(3, kind, synth.storage(w, x), threads=8)
    so = O.calibrate(x, op, 3, kind)
    sl = O.parse_artifact(c.save()).slots[(3, kind)]
    _compare_slots(sl, so)
    assert np.array_equal(sl.widths, so.widths)


def test_calibration_matches_oracle_group32_small():
    x, _ = pins.family_b_small(seed=21, n=3000)
    op = O.Params(2, 2, 32, 4, 8, 32, 8, 1.5, O.DTYPE_F32)
    kp = K.params(2, 2, 32, 4, 8, 32, 8, 1.5, K.KVTC_F32)
    c = K.Codec(kp)
    c.calibrate(1, 1, x, threads=2)
    so = O.calibrate(x, op, 1, 1)
    _compare_slots(O.parse_artifact(c.save()).slots[(1, 1)], so)


def test_artifact_bytes_interoperate():
    w = synth.workload("tiny")
    op, kp = _params_pair(w)
    x = synth.gen_kv(w, 0, 0, 1, w.calib_tokens)
    so = O.calibrate(x, op, 0, 0)
    art = O.Artifact(op, {(0, 0): so}).serialize()
    c = K.Codec.load(art)
    assert c.save() == art                       # oracle -> library -> bytes
    info = c.slot(0, 0)
    assert info.slot_id == so.slot_id and info.record_bytes == so.record_bytes
    assert list(info.widths[: op.n_groups]) == so.widths.tolist()
    c2 = K.Codec(kp)
    c2.calibrate(0, 0, synth.storage(w, x))
    back = O.parse_artifact(c2.save())         # library -> oracle parser
    assert back.slots[(0, 0)].slot_id == c2.slot(0, 0).slot_id


def test_artifact_corruption_is_rejected():
    w = synth.workload("tiny")
    op, _ = _params_pair(w)
    so = O.calibrate(synth.gen_kv(w, 0, 0, 1, 600), op, 0, 0)
    art = bytearray(O.Artifact(op, {(0, 0): so}).serialize())
    for off in (0, 4, 60, len(art) - 30, len(art) - 1):
        bad = bytearray(art)
        bad[off] ^= 0x40
        with pytest.raises(K.KvtcError) as e:
            K.Codec.load(bytes(bad))
        assert e.value.status in (K.KVTC_E_CORRUPT, K.KVTC_E_INVALID)
    with pytest.raises(K.KvtcError):
        K.Codec.load(bytes(art[:-9]))


def test_encoded_bytes_match_oracle():
    w = synth.workload("tiny")
    op, _ = _params_pair(w)
    so = O.calibrate(synth.gen_kv(w, 0, 0, 1, 800), op, 0, 0)
    c = K.Codec.load(O.Artifact(op, {(0, 0): so}).serialize())
    for T in (0, 1, 4, 5, 67, 68, 69, 512, 1000):
        assert c.encoded_bytes(0, 0, T) == O.stream_bytes(op, so, T)
    assert c.encoded_bytes(0, 1, 100) == 0          # V never calibrated


def test_bad_params_rejected():
    good = dict(n_layers=1, kv_heads=2, head_dim=64, sink=4, window=8, group=16, max_bits=8,
                bits_per_value=1.0, dtype=K.KVTC_BF16)
    for key, val in (("group", 12), ("group", 24), ("head_dim", 60), ("max_bits", 9),
                     ("bits_per_value", -1.0), ("dtype", 5), ("n_layers", 0), ("sink", -1)):
        p = dict(good, **{key: val})
        with pytest.raises(K.KvtcError) as e:
            K.kvtc_create(K.params(**p))
        assert e.value.status == K.KVTC_E_INVALID, (key, val)


def test_calibrate_errors():
    c = K.Codec(K.params(2, 1, 64, 4, 8, 16, 8, 2.0, K.KVTC_F32))
    with pytest.raises(K.KvtcError):
        c.calibrate(0, 0, np.zeros((12, 64), np.float32))       # no row after s + w
    with pytest.raises(K.KvtcError):
        c.calibrate(2, 0, np.zeros((100, 64), np.float32))      # bad layer
    with pytest.raises(K.KvtcError):
        c.calibrate(0, 2, np.zeros((100, 64), np.float32))      # bad kind


def test_job_checks_precede_any_launch():
    """Host validation (no device here): an uncalibrated slot, a src or dst
    too small, or a missing workspace is rejected before the device state is
    looked at, so nothing is launched; with valid jobs the missing upload is
    the error."""
    w = synth.workload("tiny")
    op, kp = _params_pair(w)
    c = K.Codec(kp)
    T, F = 100, w.features
    rows = T * F * 4
    job = K.make_job(0, 0, T, 4096, 8192, 1 << 20, src_capacity=rows)
    with pytest.raises(K.KvtcError) as e:
        c.encode([job], 256)
    assert e.value.status == K.KVTC_E_NOT_CALIBRATED
    c.calibrate(0, 0, synth.storage(w, synth.gen_kv(w, 0, 0, 1, w.calib_tokens)), threads=2)
    n = c.encoded_bytes(0, 0, T)
    with pytest.raises(K.KvtcError) as e:                # encode reads n_tokens rows of src
        c.encode([K.make_job(0, 0, T, 4096, 8192, n, src_capacity=rows - 16)], 256)
    assert e.value.status == K.KVTC_E_CAPACITY and "src_capacity" in str(e.value)
    with pytest.raises(K.KvtcError) as e:                # and writes the whole stream
        c.encode([K.make_job(0, 0, T, 4096, 8192, n - 1, src_capacity=rows)], 256)
    assert e.value.status == K.KVTC_E_CAPACITY
    dec = lambda cap: [K.make_job(0, 0, T, 4096, 8192, rows, src_capacity=cap)]
    with pytest.raises(K.KvtcError) as e:                # decode reads the whole stream
        c.decode(dec(n - 1), K.KVTC_F32, 256, K.kvtc_workspace_bytes(1))
    assert e.value.status == K.KVTC_E_CAPACITY and "src_capacity" in str(e.value)
    with pytest.raises(K.KvtcError) as e:
        c.encode([K.make_job(0, 0, T, 4096, 8192, n, src_capacity=rows)], 256)
    assert e.value.status == K.KVTC_E_INVALID and "kvtc_upload" in str(e.value)   # never uploaded
    with pytest.raises(K.KvtcError) as e:
        c.encode([job], 0)
    assert e.value.status == K.KVTC_E_INVALID           # no workspace
    with pytest.raises(ValueError):                      # a raw pointer needs its capacity
        K.make_job(0, 0, T, 4096, 8192, rows)


def test_zero_allocation_when_budget_too_small():
    x, _ = pins.family_b_small(seed=5, n=500)
    c = K.Codec(K.params(1, 2, 32, 4, 8, 16, 8, 79.0 / 64, K.KVTC_F32))   # 79 bits < 80
    c.calibrate(0, 0, x)
    info = c.slot(0, 0)
    assert info.n_act == 0 and info.record_bytes == 0


def test_deflate_roundtrip():
    data = bytes(np.random.default_rng(0).integers(0, 4, 50000, dtype=np.uint8))
    z = K.kvtc_deflate(data, 6)
    assert zlib.decompress(z) == data and len(z) < len(data)


def test_decode_workspace_sizes():
    """kvtc_decode_workspace_bytes: the status words and the sink, then the
    two-stage schedule's staging (0 is reserved for jobs naming an unknown or
    uncalibrated (layer, kind)); the staging is one block of ks * 1024 + 128
    bytes per 32 compressed tokens, 0 without compressed rows."""
    w = synth.workload("tiny")
    _, kp = _params_pair(w)
    c = K.Codec(kp)
    c.calibrate(0, 0, synth.storage(w, synth.gen_kv(w, 0, 0, 1, w.calib_tokens)), threads=2)
    info = c.slot(0, 0)
    ks = (info.r_eff + 15) // 16
    short = [K.make_job(0, 0, T, 16, 16, 1 << 20, src_capacity=1 << 20) for T in (0, 1, w.sink + w.window)]
    base = K.kvtc_workspace_bytes(len(short))
    assert c.staging_bytes(short) == 0
    assert c.decode_workspace_bytes(short) == base
    T = w.sink + w.window + 33                     # 33 compressed rows: two blocks
    jobs = short + [K.make_job(0, 0, T, 16, 16, 1 << 20, src_capacity=1 << 20)]
    blocks = 256 * ((2 * (ks * 1024 + 128) + 255) // 256)
    assert c.staging_bytes(jobs) == blocks
    assert c.decode_workspace_bytes(jobs) == K.kvtc_workspace_bytes(len(jobs)) + blocks
    assert c.decode_workspace_bytes([K.make_job(0, 1, T, 16, 16, 1 << 20, src_capacity=1 << 20)]) == 0   # V never calibrated


# ------------------------------------------------- calibration of a tensor set

def _set_inputs(wname="llama31_8b", layers=(0, 1), n=3000):
    w = synth.workload(wname)
    return w, [(l, k, synth.gen_kv(w, l, k, 1, n)) for l in layers for k in (0, 1)]


def _lib_set(kp, w, inputs, flags):
    c = K.Codec(kp)
    c.calibrate_set([(l, k, synth.storage(w, x)) for l, k, x in inputs], flags, threads=8)
    return c, O.parse_artifact(c.save()).slots


def _compare_set(lib_slots, orc_slots, G):
    """Library vs oracle for a set: means bit for bit, eigenvalues, the
    projector of each active group; the widths equal, or (a near tie in the
    two D tables) the same total objective within 1e-9."""
    keys = sorted(orc_slots)
    assert sorted(lib_slots) == keys
    same = all(np.array_equal(lib_slots[k].widths, orc_slots[k].widths) for k in keys)
    if not same:
        obj = lambda ws: sum(orc_slots[k].D[g, b] for k in keys for g, b in enumerate(ws[k]))
        a = obj({k: lib_slots[k].widths for k in keys})
        b = obj({k: orc_slots[k].widths for k in keys})
        assert abs(a - b) <= 1e-9 * b, (a, b)
    for k in keys:
        sl, so = lib_slots[k], orc_slots[k]
        assert np.array_equal(sl.mu32, so.mu32)
        ok = so.lam > so.lam[0] * 1e-12
        assert np.allclose(sl.lam[ok], so.lam[ok], rtol=1e-6)
        if same:
            for a, g in enumerate(so.active_groups):
                Vl = sl.V32[:, a * G:(a + 1) * G].astype(np.float64)
                Vo = so.V64[:, g * G:(g + 1) * G]
                assert np.abs(Vl @ Vl.T - Vo @ Vo.T).max() <= 1e-5, (k, g)
    return same


def test_calibrate_set_without_flags_is_per_tensor():
    w, ins = _set_inputs(n=2500)
    op, kp = _params_pair(w)
    c1, _ = _lib_set(kp, w, ins, 0)
    c2 = K.Codec(kp)
    for l, k, x in ins:
        c2.calibrate(l, k, synth.storage(w, x), threads=8)
    assert c1.save() == c2.save()


@pytest.mark.parametrize("flags", [K.KVTC_CAL_SHARED_BASIS, K.KVTC_CAL_GLOBAL_BUDGET,
                                   K.KVTC_CAL_SHARED_BASIS | K.KVTC_CAL_GLOBAL_BUDGET])
def test_calibrate_set_matches_oracle_llama8b(flags):
    w, ins = _set_inputs()
    op, kp = _params_pair(w)
    _, lib = _lib_set(kp, w, ins, flags)
    orc = O.calibrate_set(ins, op, shared_basis=bool(flags & K.KVTC_CAL_SHARED_BASIS),
                          global_budget=bool(flags & K.KVTC_CAL_GLOBAL_BUDGET),
                          max_active=K.KVTC_MAX_REFF // w.group)
    _compare_set(lib, orc, w.group)
    bits = sum(16 * int(b) + (64 if b else 0) for sl in lib.values() for b in sl.widths)
    assert bits <= len(ins) * op.budget_bits
    if flags & K.KVTC_CAL_SHARED_BASIS:
        for k in (0, 1):
            assert np.array_equal(lib[(0, k)].lam, lib[(1, k)].lam)
    if flags & K.KVTC_CAL_GLOBAL_BUDGET:   # never worse than a budget per tensor
        per = O.calibrate_set(ins, op, shared_basis=bool(flags & K.KVTC_CAL_SHARED_BASIS))
        obj = lambda sl_w, key: sum(orc[key].D[g, b] for g, b in enumerate(sl_w))
        assert sum(obj(lib[k].widths, k) for k in orc) <= sum(obj(per[k].widths, k) for k in orc) * (1 + 1e-12)


def test_calibrate_set_global_exact_small():
    """Three small tensors of very different energy, group 16 and 32: the
    library's global widths are the oracle's."""
    for G in (16, 32):
        ins = pins.three_scaled_tensors()
        op = O.Params(2, 2, 32, 4, 8, G, 8, 2.0, O.DTYPE_F32)
        kp = K.params(2, 2, 32, 4, 8, G, 8, 2.0, K.KVTC_F32)
        c = K.Codec(kp)
        c.calibrate_set(ins, K.KVTC_CAL_GLOBAL_BUDGET | K.KVTC_CAL_SHARED_BASIS, threads=2)
        lib = O.parse_artifact(c.save()).slots
        orc = O.calibrate_set(ins, op, shared_basis=True, global_budget=True, max_active=256 // G)
        assert _compare_set(lib, orc, G)


def test_calibrate_set_errors_leave_codec_unchanged():
    w, ins = _set_inputs(wname="tiny", layers=(0,), n=600)
    ins = ins[:1]
    op, kp = _params_pair(w)
    c = K.Codec(kp)
    c.calibrate(0, 0, synth.storage(w, ins[0][2]), threads=2)
    before = c.save()
    x = synth.storage(w, ins[0][2])
    for args, flags in (([(0, 0, x), (0, 0, x)], 0),            # duplicate
                        ([(0, 0, x)], 8),                          # unknown flag
                        ([(0, 0, x[: w.sink + w.window])], 0),     # no row after sink and window
                        ([(0, 0, x), (5, 0, x)], 0)):              # bad layer
        with pytest.raises(K.KvtcError) as e:
            c.calibrate_set(args, flags)
        assert e.value.status == K.KVTC_E_INVALID
        assert c.save() == before


def test_lossless_bound_matches_oracle():
    """The library's container bound and the oracle's agree on every shape of
    the lossless pins (no device needed), and an uncalibrated slot has none."""
    import oracle.kvtc_lossless as LZ
    for p, sl, T, _ in pins.lossless_streams():
        c = K.Codec.load(O.Artifact(p, {(0, 0): sl}).serialize())
        assert c.lossless_bound(0, 0, T) == LZ.container_bound(p, sl, T), (p, T)
        job = K.make_job(0, 0, T, 16, 16, 1 << 30, src_capacity=1 << 30)
        assert c.lossless_workspace_bytes([job], True) > 0 and c.lossless_workspace_bytes([job], False) > 0
    assert c.lossless_bound(0, 1, 100) == 0


def test_component_widths_match_oracle():
    """KVTC_CAL_COMPONENT_WIDTHS against the oracle's reading Q2c: small
    family-B tensors at G = 16 and 32 (widths exact), a llama31_8b tensor
    (widths, or the objective on a near tie); the artifact bytes go both
    ways; with the global budget the call is refused."""
    for G, bpv in ((16, 3.0), (32, 2.0)):
        x, _ = pins.family_b_small(seed=29, n=2200)
        op = O.Params(2, 2, 32, 4, 8, G, 8, bpv, O.DTYPE_F32)
        kp = K.params(2, 2, 32, 4, 8, G, 8, bpv, K.KVTC_F32)
        c = K.Codec(kp)
        c.calibrate_set([(1, 0, x)], K.KVTC_CAL_COMPONENT_WIDTHS, threads=2)
        so = O.calibrate_set([(1, 0, x)], op, component_widths=True)[(1, 0)]
        sl = O.parse_artifact(c.save()).slots[(1, 0)]
        assert np.array_equal(sl.cwidths, so.cwidths), (G, sl.cwidths, so.cwidths)
        assert sl.record_bytes == so.record_bytes == c.slot(1, 0).record_bytes
        assert c.slot(1, 0).per_component == 1
        art = O.Artifact(op, {(1, 0): so}).serialize()
        assert K.Codec.load(art).save() == art
    w, ins = _set_inputs(layers=(0,), n=3000)
    op, kp = _params_pair(w)
    c = K.Codec(kp)
    c.calibrate_set([(l, k, synth.storage(w, x)) for l, k, x in ins], K.KVTC_CAL_COMPONENT_WIDTHS, threads=8)
    lib = O.parse_artifact(c.save()).slots
    orc = O.calibrate_set(ins, op, component_widths=True)
    for k in orc:
        a, b = lib[k], orc[k]
        if not np.array_equal(a.cwidths, b.cwidths):
            obj = lambda cw: sum(b.D[j, v] for j, v in enumerate(cw))
            assert abs(obj(a.cwidths) - obj(b.cwidths)) <= 1e-9 * obj(b.cwidths)
        assert np.array_equal(a.mu32, b.mu32)
        assert sum(64 + 8 * ((int(s) + 7) // 8) for s in a.cwidths.reshape(-1, w.group).sum(axis=1) if s) \
            <= op.budget_bits
    with pytest.raises(K.KvtcError) as e:
        c.calibrate_set([(0, 0, synth.storage(w, ins[0][2]))],
                        K.KVTC_CAL_COMPONENT_WIDTHS | K.KVTC_CAL_GLOBAL_BUDGET)
    assert e.value.status == K.KVTC_E_INVALID


def test_allocation_keeps_to_the_kernels_cap():
    """At 8 bits per value the DP's optimum on a llama31_8b tensor wants more
    than KVTC_MAX_REFF components; the library keeps to the cap with the
    allocation that is optimal under both limits, the oracle's capped one."""
    w = synth.workload("llama31_8b")
    x = synth.gen_kv(w, 0, 0, 1, 2000)
    op = O.Params(w.n_layers, w.kv_heads, w.head_dim, w.sink, w.window, w.group, 8, 8.0, O.DTYPE_BF16)
    kp = K.params(w.n_layers, w.kv_heads, w.head_dim, w.sink, w.window, w.group, 8, 8.0, K.KVTC_BF16)
    cap = K.KVTC_MAX_REFF // w.group
    free = O.calibrate(x, op, 0, 0)
    assert free.n_act > cap                     # the uncapped optimum needs more
    so = O.calibrate(x, op, 0, 0, max_active=cap)
    c = K.Codec(kp)
    c.calibrate(0, 0, synth.storage(w, x), threads=8)
    sl = O.parse_artifact(c.save()).slots[(0, 0)]
    assert sl.n_act <= cap and so.n_act <= cap
    _compare_slots(sl, so)


@pytest.mark.parametrize("name", ["llama31_8b", "offsets_bf16", "odd1_f32"])
def test_folded_mean_follows_the_documented_bound(name):
    """The encode folds the mean into the product exactly for bf16 slots with
    |mu32|^2 <= sum of the covariance eigenvalues (kvtc_slot_info.folded_mean);
    checked on oracle-calibrated slots: a Llama-shaped layer (mean about half
    the spread: folded), one with offsets far above the spread and an f32
    tensor (both centred)."""
    w = synth.workload(name)
    op, _ = _params_pair(w)
    n = min(w.calib_tokens, 4096)
    slots = {(0, k): O.calibrate(synth.gen_kv(w, 0, k, 1, n), op, 0, k) for k in range(len(w.kinds))}
    c = K.Codec.load(O.Artifact(op, slots).serialize())
    for (l, k), so in slots.items():
        expect = (op.dtype == O.DTYPE_BF16 and so.r_eff > 0
                  and float(np.sum(so.mu32.astype(np.float64) ** 2)) <= float(np.sum(so.lam)))
        assert c.slot(l, k).folded_mean == int(expect)
        if name == "llama31_8b":
            assert expect
        else:
            assert not expect


def test_component_widths_keep_to_the_kernels_cap():
    """A width per component at 8 bits per value on 10 groups of 32: the plain
    allocation wants more than KVTC_MAX_REFF / 32 = 8 active groups; the
    library keeps to the cap with the oracle's capped allocation (reading
    Q3c), equal widths or an equal objective on a near tie."""
    rng = np.random.default_rng(41)
    F, G, n = 320, 32, 2000
    Q = np.linalg.qr(rng.standard_normal((F, F)))[0]
    x = ((rng.standard_normal((n, F)) * np.linspace(3.0, 0.5, F)) @ Q.T).astype(np.float32)
    op = O.Params(1, 5, 64, 4, 8, G, 8, 8.0, O.DTYPE_F32)
    kp = K.params(1, 5, 64, 4, 8, G, 8, 8.0, K.KVTC_F32)
    cap = K.KVTC_MAX_REFF // G
    free = O.calibrate_set([(0, 0, x)], op, component_widths=True)[(0, 0)]
    assert free.n_act > cap                     # the plain optimum needs more
    so = O.calibrate_set([(0, 0, x)], op, component_widths=True, max_active=cap)[(0, 0)]
    assert so.n_act <= cap
    c = K.Codec(kp)
    c.calibrate_set([(0, 0, x)], K.KVTC_CAL_COMPONENT_WIDTHS, threads=8)
    sl = O.parse_artifact(c.save()).slots[(0, 0)]
    assert sl.n_act <= cap
    if not np.array_equal(sl.cwidths, so.cwidths):   # a near tie may flip
        obj = lambda cw: sum(so.D[j, b] for j, b in enumerate(cw))
        assert abs(obj(sl.cwidths) - obj(so.cwidths)) <= 1e-9 * obj(so.cwidths)
