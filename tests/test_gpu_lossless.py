"""The GPU lossless stage (cuda:0, through the C ABI) against the oracle's
container, byte for byte, and its inverse.

The KVTC page (section 2B) ends compression with DEFLATE on the GPU; the
library's lossless stage is a per-field static rANS coder of its own
(format in include/kvtc.h). Integer work: every container must equal the
oracle's bytes exactly, and decoding must give the stream back exactly."""
import zlib

import numpy as np
import pytest
import torch

import kv_cache_transform_amd as K
import oracle.kvtc_lossless as LZ
import oracle.kvtc_oracle as O
import pins
import synth
from gpu_util import DEV, DevCodec, oracle_artifact, oracle_params, to_dev_bytes

pytestmark = pytest.mark.gpu


def _streams(wname, slots, T, calib=None):
    art = oracle_artifact(wname, slots, calib)
    w = synth.workload(wname)
    out = []
    for l, k in slots:
        store = synth.storage(w, synth.gen_kv(w, l, k, synth.ROLE_EVAL, T))
        out.append((l, k, T, O.encode(store, art.params, art.slots[(l, k)], l, k).stream))
    return art, out


def _run(art, items, src_pad=0):
    """items: (layer, kind, T, stream bytes). Lossless encode on the GPU, the
    sizes, the containers (bytes), and the streams decoded back."""
    dc = DevCodec(art.serialize())
    c = dc.codec
    srcs = [to_dev_bytes(st, 16) for _, _, _, st in items]
    bounds = [c.lossless_bound(l, k, T) for l, k, T, _ in items]
    dsts = [torch.full((b + 16,), 0xA5, dtype=torch.uint8, device=DEV) for b in bounds]
    jobs = [K.make_job(l, k, T, s, d, b, src_capacity=len(st))
            for (l, k, T, st), s, d, b in zip(items, srcs, dsts, bounds)]
    n = K.kvtc_lossless_workspace_bytes(c.h, jobs, True)
    ws = torch.zeros(n, dtype=torch.uint8, device=DEV)
    stream = torch.cuda.current_stream()
    c.lossless_encode(jobs, ws, n, stream)
    st = K.kvtc_read_device_status(ws, len(jobs), stream)
    assert np.all(st == 0), st
    sizes = K.kvtc_lossless_sizes(ws, len(jobs), stream)
    conts = [bytes(d[:int(z)].cpu().numpy().tobytes()) for d, z in zip(dsts, sizes)]
    back = _decode(c, [(l, k, T, z, len(stb)) for (l, k, T, stb), z in zip(items, conts)], src_pad)
    return conts, back


def _decode(c, items, src_pad=0, fill=0x5C):
    """items: (layer, kind, T, container bytes, stream bytes)."""
    srcs = [to_dev_bytes(z, src_pad) for _, _, _, z, _ in items]
    dsts = [torch.full((max(nb, 16),), fill, dtype=torch.uint8, device=DEV) for *_, nb in items]
    jobs = [K.make_job(l, k, T, s, d, nb, src_capacity=len(z) + src_pad)
            for (l, k, T, z, nb), s, d in zip(items, srcs, dsts)]
    n = K.kvtc_lossless_workspace_bytes(c.h, jobs, False)
    ws = torch.zeros(n, dtype=torch.uint8, device=DEV)
    stream = torch.cuda.current_stream()
    c.lossless_decode(jobs, ws, n, stream)
    st = K.kvtc_read_device_status(ws, len(jobs), stream)
    return st, [bytes(d[:nb].cpu().numpy().tobytes()) for d, (*_, nb) in zip(dsts, items)]


CASES = {
    "tiny": ("tiny", [(0, 0)], 512, None),
    "odd3_bf16": ("odd3_bf16", [(0, 0), (0, 1)], 1100, None),
    "odd1_f32": ("odd1_f32", [(0, 0)], 2100, None),
    "llama31_8b": ("llama31_8b", [(0, 0), (0, 1), (1, 0)], 8192, 4096),
    "nemo12b_g32": ("nemo12b", [(0, 0)], 6000, 4096),
}


@pytest.mark.parametrize("case", list(CASES))
def test_lossless_matches_oracle(case):
    wname, slots, T, calib = CASES[case]
    art, items = _streams(wname, slots, T, calib)
    conts, (st, back) = _run(art, items)
    assert np.all(st == 0), st
    raw = len(items) * T * art.params.F * art.params.elem_bytes
    tot_z = tot_s = tot_d = 0
    for (l, k, T_, stb), z, b in zip(items, conts, back):
        ref = LZ.compress(stb, art.params, art.slots[(l, k)], T_)
        assert len(z) == len(ref)
        assert z == ref, "container differs from the oracle's"
        assert b == stb, "decoded stream differs"
        tot_z += len(z)
        tot_s += len(stb)
        tot_d += len(zlib.compress(stb, 6))
    print(f"{case}: raw/stream {raw / tot_s:.3f} raw/container {raw / tot_z:.3f} raw/zlib {raw / tot_d:.3f}")


def _pc_streams(wname, slots, T, calib, mixed):
    """Streams of slots with a width per component (the oracle's reading
    Q2c); with mixed, every width 0..8 inside each active group."""
    w = synth.workload(wname)
    op = oracle_params(w)
    ins = [(l, k, synth.gen_kv(w, l, k, synth.ROLE_CALIB, calib or w.calib_tokens)) for l, k in slots]
    sls = O.calibrate_set(ins, op, component_widths=True)
    if mixed:
        for sl in sls.values():
            cw = sl.cwidths.copy()
            for a, g in enumerate(sl.active_groups):
                cw[g * sl.G:(g + 1) * sl.G] = [(3 * a + 5 * i + 1) % 9 for i in range(sl.G)]
                cw[g * sl.G] = max(cw[g * sl.G], 1)
            sl.cwidths = cw
            sl.widths = cw.reshape(-1, sl.G).max(axis=1).astype(np.uint8)
    art = O.Artifact(op, sls)
    items = []
    for l, k in slots:
        store = synth.storage(w, synth.gen_kv(w, l, k, synth.ROLE_EVAL, T))
        items.append((l, k, T, O.encode(store, op, art.slots[(l, k)], l, k).stream))
    return art, items


PC_CASES = {
    "llama31_8b_mixed": ("llama31_8b", [(0, 0), (0, 1)], 8192, 4096, True),
    "nemo12b_g32_mixed": ("nemo12b", [(0, 0)], 6000, 4096, True),
    "odd3_bf16": ("odd3_bf16", [(0, 0), (0, 1)], 1100, None, False),
    "odd1_f32_mixed": ("odd1_f32", [(0, 0)], 2100, None, True),
}


@pytest.mark.parametrize("case", list(PC_CASES))
def test_lossless_per_component_widths(case):
    """Streams with a width per component: the container equals the oracle's
    (reading L1c) byte for byte and decodes back to the stream."""
    art, items = _pc_streams(*PC_CASES[case])
    conts, (st, back) = _run(art, items)
    assert np.all(st == 0), st
    for (l, k, T, stb), z, b in zip(items, conts, back):
        assert z == LZ.compress(stb, art.params, art.slots[(l, k)], T), "container differs from the oracle's"
        assert b == stb, "decoded stream differs"


def test_lossless_edge_shapes():
    """Lengths 0, 1, all passthrough, one compressed row and a ragged last
    chunk; every width 1..8 on one injected slot; no active group; f32 and
    bf16; all in one call per artifact."""
    streams = pins.lossless_streams()
    by_art = {}
    for p, sl, T, st in streams:
        cw = None if sl.cwidths is None else tuple(sl.cwidths.tolist())
        key = (p.F, p.group, p.dtype, tuple(sl.widths.tolist()), cw, float(np.sum(sl.V32)))
        by_art.setdefault(key, (p, sl, []))[2].append((T, st))
    for p, sl, lst in by_art.values():
        art = O.Artifact(p, {(0, 0): sl})
        items = [(0, 0, T, st) for T, st in lst]
        conts, (stt, back) = _run(art, items)
        assert np.all(stt == 0), stt
        for (_, _, T, stb), z, b in zip(items, conts, back):
            assert z == LZ.compress(stb, p, sl, T), T
            assert b == stb, T


def test_lossless_many_jobs_two_launches():
    """40 jobs (two launches of the lossless kernels) of mixed lengths."""
    wname = "odd3_bf16"
    art = oracle_artifact(wname, [(0, 0), (0, 1)])
    w = synth.workload(wname)
    items = []
    for i in range(40):
        l, k, T = 0, i % 2, [0, 1, 70, 300, 1100][i % 5]
        store = synth.storage(w, synth.gen_kv(w, l, k, synth.ROLE_EVAL, max(T, 1)))[:T]
        items.append((l, k, T, O.encode(store, art.params, art.slots[(l, k)], l, k).stream))
    conts, (st, back) = _run(art, items)
    assert np.all(st == 0), st
    for (l, k, T, stb), z, b in zip(items, conts, back):
        assert z == LZ.compress(stb, art.params, art.slots[(l, k)], T)
        assert b == stb


def test_lossless_bad_containers_write_nothing():
    """A container that does not belong to the job's shape (MISMATCH), one
    whose payload is damaged or larger than src_capacity says (CORRUPT): the
    job's status says so and its stream buffer keeps its fill; the good job
    in the same call decodes."""
    art, items = _streams("odd3_bf16", [(0, 0), (0, 1)], 1100)
    (l0, k0, T0, s0), (l1, k1, T1, s1) = items
    z0 = LZ.compress(s0, art.params, art.slots[(l0, k0)], T0)
    z1 = LZ.compress(s1, art.params, art.slots[(l1, k1)], T1)
    bad = bytearray(z0)
    pay = int(np.frombuffer(z0, "<u4", 1, 32)[0])
    bad[pay] ^= 0x5A                                   # low word of chunk 0's final state
    with pytest.raises(O.OracleError):
        LZ.decompress(bytes(bad), art.params, art.slots[(l0, k0)], T0)
    dc = DevCodec(art.serialize())
    c = dc.codec
    cases = [((l0, k0, T0, bytes(bad), len(s0)), K.KVTC_E_CORRUPT),
             ((l1, k1, T1 + 1, z1, c.encoded_bytes(l1, k1, T1 + 1)), K.KVTC_E_MISMATCH),
             ((l0, k0, T0, z0, len(s0)), K.KVTC_OK)]
    st, outs = _decode(c, [it for it, _ in cases])
    assert st.tolist() == [want for _, want in cases], st
    assert outs[0] == bytes([0x5C]) * len(outs[0]) and outs[1] == bytes([0x5C]) * len(outs[1])
    assert outs[2] == s0
    # the container claims more bytes than src_capacity allows
    z_short = (l0, k0, T0, z0[:-16], len(s0))
    st, outs = _decode(c, [z_short])
    assert st.tolist() == [K.KVTC_E_CORRUPT] and outs[0] == bytes([0x5C]) * len(outs[0])


def test_lossless_host_checks():
    art, items = _streams("tiny", [(0, 0)], 512)
    dc = DevCodec(art.serialize())
    c = dc.codec
    l, k, T, st = items[0]
    src = to_dev_bytes(st, 16)
    b = c.lossless_bound(l, k, T)
    dst = torch.zeros(b, dtype=torch.uint8, device=DEV)
    job = K.make_job(l, k, T, src, dst, b, src_capacity=len(st))
    n = K.kvtc_lossless_workspace_bytes(c.h, [job], True)
    ws = torch.zeros(n, dtype=torch.uint8, device=DEV)
    with pytest.raises(K.KvtcError) as e:
        c.lossless_encode([job], ws, n - 256)
    assert e.value.status == K.KVTC_E_CAPACITY
    with pytest.raises(K.KvtcError) as e:
        c.lossless_encode([K.make_job(l, k, T, src, dst, b - 1, src_capacity=len(st))], ws, n)
    assert e.value.status == K.KVTC_E_CAPACITY
