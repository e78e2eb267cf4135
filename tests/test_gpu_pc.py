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
