"""A width per component inside each microscale group (cuda:0, through the
C ABI), against the oracle's reading Q2c: artifacts calibrated by the oracle
with component_widths, streams encoded by the library, codes and records
compared with the oracle's, and the oracle's streams decoded by the
two-stage and fused schedules and by kvtc_decode_noalloc."""
import functools

import numpy as np
import pytest
import torch

import kv_cache_transform_amd as K
import oracle.kvtc_oracle as O
import synth
from gpu_util import DEV, DevCodec, bf16_out_to_f64, code_stats, oracle_params, storage_to_dev, to_dev_bytes

pytestmark = pytest.mark.gpu

CODE_RATE = 1e-4
DEC_TOL = 1e-3

# name: (workload, slots, T, calibration tokens)
CASES = {
    "llama31_8b": ("llama31_8b", [(0, 0), (0, 1)], 8192, 4096),
    # the same slots with every width 0..8 mixed inside each active group
    # (the calibration gives equal widths there: the spectrum is smooth)
    "llama31_8b_mixed": ("llama31_8b", [(0, 0), (0, 1)], 8192, 4096),
    "nemo12b_g32": ("nemo12b", [(0, 0)], 6000, 4096),
    "odd3_bf16": ("odd3_bf16", [(0, 0), (0, 1)], 1100, None),
    "odd1_f32": ("odd1_f32", [(0, 0)], 2100, None),
}


@functools.lru_cache(maxsize=None)
def _setup(case):
    wname, slots, T, calib = CASES[case]
    w = synth.workload(wname)
    op = oracle_params(w)
    n = calib or w.calib_tokens
    ins = [(l, k, synth.gen_kv(w, l, k, synth.ROLE_CALIB, n)) for l, k in slots]
    slots_pc = O.calibrate_set(ins, op, component_widths=True)
    if case.endswith("_mixed"):
        for sl in slots_pc.values():
            cw = sl.cwidths.copy()
            for a, g in enumerate(sl.active_groups):
                cw[g * sl.G:(g + 1) * sl.G] = [(3 * a + 5 * i + 1) % 9 for i in range(sl.G)]
                cw[g * sl.G] = max(cw[g * sl.G], 1)     # the group stays active
            sl.cwidths = cw
            sl.widths = cw.reshape(-1, sl.G).max(axis=1).astype(np.uint8)
    art = O.Artifact(op, slots_pc)
    items = []
    for l, k in slots:
        store = synth.storage(w, synth.gen_kv(w, l, k, synth.ROLE_EVAL, T))
        items.append((l, k, store, O.encode(store, op, art.slots[(l, k)], l, k)))
    return w, art, op, items


@pytest.mark.parametrize("case", list(CASES))
def test_pc_encode_parity(case):
    w, art, op, items = _setup(case)
    assert all(sl.cwidths is not None for sl in art.slots.values())
    mixed = any(len(set(sl.group_cwidths(g).tolist())) > 1
                for sl in art.slots.values() for g in sl.active_groups)
    assert mixed or not case.endswith("_mixed")
    dc = DevCodec(art.serialize())
    streams = dc.encode([(l, k, storage_to_dev(store)) for l, k, store, _ in items])
    bad = total = worst = 0
    for (l, k, store, ref), sb in zip(items, streams):
        slot = art.slots[(l, k)]
        T = store.shape[0]
        assert len(sb) == len(ref.stream)
        s1, w1, tc = O.split_rows(T, op.sink, op.window)
        rec0 = O.HEADER_BYTES + (s1 + w1) * op.F * op.elem_bytes
        assert sb[:rec0] == ref.stream[:rec0], "header or passthrough differs"
        nb, nt, mx, shift, scale = code_stats(sb, ref, op, slot, T)
        bad, total, worst = bad + nb, total + nt, max(worst, mx)
        gcodes, gshift, gscale = O.read_records(sb, op, slot, T)
        assert O.build_records(gcodes, gshift, gscale, slot).tobytes() == sb[rec0:]
        assert np.allclose(shift, ref.shift, rtol=1e-5, atol=1e-6 * np.abs(ref.shift).max())
    rate = bad / max(total, 1)
    print(f"{case}: code mismatches {bad}/{total} = {rate:.2e}, max step {worst}")
    assert worst <= 1 and rate <= CODE_RATE


@pytest.mark.parametrize("out_dtype", [K.KVTC_F32, K.KVTC_BF16])
@pytest.mark.parametrize("case", list(CASES))
def test_pc_decode_parity(case, out_dtype):
    w, art, op, items = _setup(case)
    dc = DevCodec(art.serialize())
    T = items[0][2].shape[0]
    jobs = [(l, k, T, ref.stream) for l, k, _, ref in items]
    outs, st = dc.decode(jobs, out_dtype, op.F, schedule="staged")
    assert np.all(st == 0), st
    worst = 0.0
    for (l, k, store, ref), out in zip(items, outs):
        full, ref_out = O.decode(ref.stream, op, art.slots[(l, k)], l, k, T, out_dtype)
        g = out[:T].cpu().numpy().astype(np.float64) if out_dtype == K.KVTC_F32 else bf16_out_to_f64(out[:T])
        M = max(np.abs(full).max(), 1e-30)
        err = np.abs(g - full)
        if out_dtype == K.KVTC_F32:
            assert err.max() / M <= DEC_TOL
        else:
            assert np.all(err <= DEC_TOL * M + 2.0 ** -8 * np.abs(full))
        worst = max(worst, err.max() / M)
    print(f"{case} out={out_dtype}: max rel err {worst:.3e}")
    outs2, st2 = dc.decode(jobs, out_dtype, op.F, two_stage=True, stg_fill=0xFF)
    assert np.all(st2 == 0)
    for a, b in zip(outs, outs2):
        assert torch.equal(a, b)
    # the fused schedule builds the same operands from the records in LDS
    outs3, st3 = dc.decode(jobs, out_dtype, op.F, schedule="fused")
    assert np.all(st3 == 0), st3
    for a, b in zip(outs, outs3):
        assert torch.equal(a, b)


def test_pc_noalloc_decodes_and_hooks_refuse():
    """kvtc_decode_noalloc (the fused schedule without a workspace) decodes
    slots with a width per component exactly as kvtc_decode does; the pack
    test hook, which takes group widths, refuses them before any launch."""
    w, art, op, items = _setup("odd3_bf16")
    dc = DevCodec(art.serialize())
    T = items[0][2].shape[0]
    ref_outs, st = dc.decode([(l, k, T, ref.stream) for l, k, _, ref in items], K.KVTC_BF16, op.F)
    assert np.all(st == 0), st
    srcs = [to_dev_bytes(ref.stream, 16) for _, _, _, ref in items]
    outs = [torch.zeros((T, op.F), dtype=torch.int16, device=DEV) for _ in items]
    jobs = [K.make_job(l, k, T, src, out, out.numel() * 2, src_capacity=len(ref.stream))
            for (l, k, _, ref), src, out in zip(items, srcs, outs)]
    d_st = torch.full((len(jobs),), -99, dtype=torch.int32, device=DEV)
    dc.codec.decode_noalloc(jobs, K.KVTC_BF16, d_st)
    torch.cuda.synchronize()
    assert d_st.cpu().tolist() == [0] * len(jobs)
    for a, b in zip(ref_outs, outs):
        assert torch.equal(a[:T], b)
    l, k, store, ref = items[0]
    x = storage_to_dev(store)
    buf = torch.zeros(len(ref.stream), dtype=torch.uint8, device=DEV)
    codes = torch.zeros(T * op.F, dtype=torch.uint8, device=DEV)
    ss = torch.zeros(T * op.F * 2, dtype=torch.float32, device=DEV)
    with pytest.raises(K.KvtcError) as e:
        dc.codec.pack(K.make_job(l, k, T, x, buf, len(ref.stream)), codes, ss, dc.ws)
    assert e.value.status == K.KVTC_E_UNSUPPORTED


def test_pc_and_group_slots_in_one_call():
    """One call over jobs of a slot with a width per component and of a slot
    with group widths, alternating: encode, both decode schedules (the host
    gives each kind launches of its own) and the lossless round trip all
    match the oracle."""
    import oracle.kvtc_lossless as LZ
    w = synth.workload("odd3_bf16")
    op = oracle_params(w)
    x0 = synth.gen_kv(w, 0, 0, synth.ROLE_CALIB, w.calib_tokens)
    x1 = synth.gen_kv(w, 0, 1, synth.ROLE_CALIB, w.calib_tokens)
    slots = {(0, 0): O.calibrate_set([(0, 0, x0)], op, component_widths=True)[(0, 0)],
             (0, 1): O.calibrate(x1, op, 0, 1)}
    art = O.Artifact(op, slots)
    dc = DevCodec(art.serialize())
    assert dc.codec.slot(0, 0).per_component == 1 and dc.codec.slot(0, 1).per_component == 0
    items = []
    for i, T in enumerate((700, 1100, 33, 900)):
        k = i % 2
        store = synth.storage(w, synth.gen_kv(w, 0, k, synth.ROLE_EVAL, T))
        items.append((k, T, store, O.encode(store, op, slots[(0, k)], 0, k)))
    streams = dc.encode([(0, k, storage_to_dev(store)) for k, _, store, _ in items])
    for (k, T, _, ref), sb in zip(items, streams):
        nb, nt, mx, _, _ = code_stats(sb, ref, op, slots[(0, k)], T)
        assert mx <= 1 and nb <= max(2, nt * CODE_RATE), (k, T, nb, nt)
    jobs = [(0, k, T, ref.stream) for k, T, _, ref in items]
    outs, st = dc.decode(jobs, K.KVTC_F32, op.F, schedule="staged")
    assert np.all(st == 0), st
    outs2, st2 = dc.decode(jobs, K.KVTC_F32, op.F, schedule="fused")
    assert np.all(st2 == 0), st2
    for (k, T, _, ref), a, b in zip(items, outs, outs2):
        assert torch.equal(a, b)
        full, _ = O.decode(ref.stream, op, slots[(0, k)], 0, k, T, K.KVTC_F32)
        g = a[:T].cpu().numpy().astype(np.float64)
        assert np.abs(g - full).max() / max(np.abs(full).max(), 1e-30) <= DEC_TOL
    # lossless: containers equal the oracle's and decode back
    srcs = [to_dev_bytes(ref.stream, 16) for *_, ref in items]
    bounds = [dc.codec.lossless_bound(0, k, T) for k, T, _, _ in items]
    dsts = [torch.zeros(b + 16, dtype=torch.uint8, device=DEV) for b in bounds]
    ljobs = [K.make_job(0, k, T, s, d, b, src_capacity=len(ref.stream))
             for (k, T, _, ref), s, d, b in zip(items, srcs, dsts, bounds)]
    n = dc.codec.lossless_workspace_bytes(ljobs, True)
    lws = torch.zeros(n, dtype=torch.uint8, device=DEV)
    dc.codec.lossless_encode(ljobs, lws, n)
    torch.cuda.synchronize()
    assert np.all(K.kvtc_read_device_status(lws, len(ljobs), None) == 0)
    sizes = K.kvtc_lossless_sizes(lws, len(ljobs), None)
    for (k, T, _, ref), d, z in zip(items, dsts, sizes):
        assert bytes(d[:int(z)].cpu().numpy().tobytes()) == LZ.compress(ref.stream, op, slots[(0, k)], T)
