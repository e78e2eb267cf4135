"""GPU parity of libkvtc against the CPU oracle (cuda:0, through the C ABI).

Contract (oracle = oracle/kvtc_oracle.py; every input is seeded and
synthetic, every artifact is written by the oracle and loaded by the library):
  T1  kvtc_pack of the oracle's codes and (shift, scale) reproduces the
      oracle's stream byte for byte; kvtc_decode_unpack of the oracle's stream
      returns its codes and fp32 bits exactly.
  T2  GPU encode codes differ from the oracle's in at most 1e-4 of positions
      (pooled per workload), each by at most one step.
  T3  GPU decode of the oracle's stream: max |x_gpu - x_orc| / max |x_orc|
      <= 1e-3 for fp32 output; bf16 output within 1e-3 * max|x| plus the bf16
      rounding of the value (2^-8 relative).
  T4  header and passthrough bytes are bit-exact.
"""
import numpy as np
import pytest
import torch

import kv_cache_transform_amd as K
import oracle.kvtc_oracle as O
import synth
from gpu_util import (DEV, DevCodec, bf16_out_to_f64, code_stats, oracle_artifact,
                      oracle_artifact_set, oracle_params, storage_to_dev, to_dev_bytes)

pytestmark = pytest.mark.gpu

CODE_RATE = 1e-4
DEC_TOL = 1e-3

# name: (workload, slots, T, requests, calibration tokens or None for the workload's)
CASES = {
    "tiny": ("tiny", [(0, 0)], 512, 1, None),
    "llama31_8b": ("llama31_8b", [(0, 0), (0, 1), (1, 0), (1, 1)], 8192, 1, None),
    "nemo12b": ("nemo12b", [(0, 0), (0, 1)], 32768, 1, 4096),
    "llama33_70b_16x": ("llama33_70b_16x", [(0, 0), (0, 1)], 16384, 1, 4096),
    "llama33_70b_64x": ("llama33_70b_64x", [(0, 0), (0, 1)], 16384, 1, 4096),
    "qwen25_7b_paged": ("qwen25_7b_paged", [(0, 0), (0, 1)], 8192, 2, 4096),
    # feature counts 192 and 64: an odd number of 64-feature slices
    "odd3_bf16": ("odd3_bf16", [(0, 0), (0, 1)], 1100, 1, None),
    "odd1_f32": ("odd1_f32", [(0, 0)], 2100, 1, None),
    # per-feature mean offsets about 40 times the spread
    "offsets_bf16": ("offsets_bf16", [(0, 0), (0, 1)], 4096, 1, None),
    # three layers x {K, V} calibrated as one set: a basis shared by the layers
    # of each kind and one bit budget over the six tensors (record sizes and
    # active groups differ per tensor)
    "llama31_8b_set": ("llama31_8b", [(l, k) for l in range(3) for k in (0, 1)], 8192, 1, 4096),
}
SET_CASES = {"llama31_8b_set": (True, True)}


def _setup(case):
    wname, slots, T, reqs, calib = CASES[case]
    w = synth.workload(wname)
    if case in SET_CASES:
        art = oracle_artifact_set(wname, tuple(slots), calib, *SET_CASES[case])
    else:
        art = oracle_artifact(wname, slots, calib)
    op = art.params
    items = []
    for (l, k) in slots:
        for r in range(reqs):
            store = synth.storage(w, synth.gen_kv(w, l, k, synth.ROLE_EVAL, T, r))
            items.append((l, k, store, O.encode(store, op, art.slots[(l, k)], l, k)))
    return w, art, op, items


def _decode_check(w, op, slot, ref_stream, T, out, out_dtype, layer, kind, rows=None):
    full, ref_out = O.decode(ref_stream, op, slot, layer, kind, T, out_dtype)
    got = out[:T] if rows is None else out[rows]
    s1, w1, tc = O.split_rows(T, op.sink, op.window)
    if out_dtype == K.KVTC_F32:
        g = got.cpu().numpy().astype(np.float64)
    else:
        g = bf16_out_to_f64(got)
    M = max(np.abs(full).max(initial=0.0), 1e-30)
    err = np.abs(g - full)
    if out_dtype == K.KVTC_F32:
        rel = err.max(initial=0.0) / M
        assert rel <= DEC_TOL, rel
    else:
        assert np.all(err <= DEC_TOL * M + 2.0 ** -8 * np.abs(full)), err.max()
        rel = err.max(initial=0.0) / M
    if out_dtype == op.dtype:  # passthrough rows come back bit for bit
        raw = got.cpu().numpy()
        ref = ref_out.view(np.int16) if ref_out.dtype == np.uint16 else ref_out
        pt = np.r_[0:s1, T - w1:T]
        assert np.array_equal(raw[pt].view(np.uint8), np.ascontiguousarray(ref[pt]).view(np.uint8))
    return rel


@pytest.mark.parametrize("case", list(CASES))
def test_encode_parity(case):
    _check_encode(case)


# A persistent encode workgroup walks a contiguous range of tiles, with the
# next tile's first slices in flight during a tile's quantization. Capping
# the grid at 8 workgroups gives each one many tiles, across job boundaries,
# with an even (llama31_8b) and an odd (odd3_bf16, odd1_f32) slice count.
@pytest.mark.parametrize("case", ["llama31_8b", "odd3_bf16", "odd1_f32"])
def test_encode_parity_few_workgroups(case, monkeypatch):
    monkeypatch.setenv("KVTC_MAX_WORKGROUPS", "8")
    _check_encode(case)


# Stage 2 is persistent too: with 8 workgroups each range crosses job and
# feature-slab boundaries (odd3_bf16 ends in a partial slab); the arithmetic
# per output element does not depend on the split, so the output is identical.
@pytest.mark.parametrize("case", ["llama31_8b", "odd3_bf16", "qwen25_7b_paged"])
def test_decode_few_workgroups_is_identical(case, monkeypatch):
    w, art, op, items = _setup(case)
    dc = DevCodec(art.serialize())
    T = items[0][2].shape[0]
    jobs = [(l, k, T, ref.stream) for l, k, _, ref in items]
    outs, st = dc.decode(jobs, K.KVTC_BF16, op.F)
    monkeypatch.setenv("KVTC_MAX_WORKGROUPS", "8")
    outs8, st8 = dc.decode(jobs, K.KVTC_BF16, op.F)
    assert np.all(st == 0) and np.all(st8 == 0), (st, st8)
    for a, b in zip(outs, outs8):
        assert torch.equal(a, b)


def _check_encode(case):
    w, art, op, items = _setup(case)
    dc = DevCodec(art.serialize())
    devs = [storage_to_dev(store) for _, _, store, _ in items]
    streams = dc.encode([(l, k, x) for (l, k, _, _), x in zip(items, devs)])
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
        # the records hold nothing but those codes and (shift, scale) pairs,
        # laid out as the oracle lays them out (no stray or misplaced bits)
        gcodes, gshift, gscale = O.read_records(sb, op, slot, T)
        assert O.build_records(gcodes, gshift, gscale, slot).tobytes() == sb[rec0:]
        if slot.n_act:
            assert np.allclose(shift, ref.shift, rtol=1e-5, atol=1e-6 * np.abs(ref.shift).max())
            assert np.allclose(scale, ref.scale, rtol=1e-4, atol=1e-6 * np.abs(ref.scale).max())
    rate = bad / max(total, 1)
    print(f"{case}: code mismatches {bad}/{total} = {rate:.2e}, max step {worst}")
    assert worst <= 1
    assert rate <= CODE_RATE


@pytest.mark.parametrize("out_dtype", [K.KVTC_F32, K.KVTC_BF16])
@pytest.mark.parametrize("case", list(CASES))
def test_decode_parity(case, out_dtype):
    w, art, op, items = _setup(case)
    dc = DevCodec(art.serialize())
    T = items[0][2].shape[0]
    paging = None
    if synth.workload(CASES[case][0]).paged:
        rng = np.random.default_rng(3)
        bs = w.block_size
        nblk = (T + bs - 1) // bs + 37
        paging, tables = [], []
        for _ in items:
            table = rng.permutation(nblk)[: (T + bs - 1) // bs].astype(np.int32)
            tables.append(table)
            paging.append((torch.from_numpy(table).to(DEV), bs, nblk))
    outs, st = dc.decode([(l, k, T, ref.stream) for l, k, _, ref in items], out_dtype, op.F, paging)
    assert np.all(st == 0), st
    worst = 0.0
    for i, (l, k, store, ref) in enumerate(items):
        rows = None
        if paging is not None:
            t = np.arange(T)
            rows = torch.from_numpy(tables[i][t // w.block_size] * w.block_size + t % w.block_size).to(DEV)
        worst = max(worst, _decode_check(w, op, art.slots[(l, k)], ref.stream, T, outs[i],
                                         out_dtype, l, k, rows))
    print(f"{case} out={out_dtype}: max rel err {worst:.3e}")
    # the two-stage path computes exactly what the fused one does, through
    # the explicit stage calls and through kvtc_decode given the staging
    for kw in ({"two_stage": True}, {"schedule": "staged", "stg_fill": 0xFF}):
        outs2, st2 = dc.decode([(l, k, T, ref.stream) for l, k, _, ref in items], out_dtype, op.F,
                               paging, **kw)
        assert np.all(st2 == 0), (kw, st2)
        for a, b in zip(outs, outs2):
            assert torch.equal(a, b), kw


@pytest.mark.parametrize("case", list(CASES))
def test_pack_unpack_bit_exact(case):
    """T1 on every workload and every tensor of its sample: kvtc_pack of the
    oracle's codes and (shift, scale) reproduces the oracle's stream byte for
    byte, and kvtc_unpack of the oracle's stream returns them bit for bit."""
    w, art, op, items = _setup(case)
    dc = DevCodec(art.serialize())
    for l, k, store, ref in items:
        slot = art.slots[(l, k)]
        T = store.shape[0]
        x = storage_to_dev(store)
        n = dc.codec.encoded_bytes(l, k, T)
        buf = torch.zeros(n, dtype=torch.uint8, device=DEV)
        codes = torch.from_numpy(np.ascontiguousarray(ref.codes)).to(DEV)
        ss = torch.from_numpy(np.ascontiguousarray(np.stack([ref.shift, ref.scale], axis=2))).to(DEV)
        job = K.make_job(l, k, T, x, buf, n)
        dc.codec.pack(job, codes, ss, dc.ws, torch.cuda.current_stream())
        torch.cuda.synchronize()
        assert bytes(buf.cpu().numpy().tobytes()) == ref.stream          # T1 pack
        src = to_dev_bytes(ref.stream, 16)
        out = torch.zeros((T, op.F), dtype=torch.int16 if op.dtype == O.DTYPE_BF16 else torch.float32,
                          device=DEV)
        djob = K.make_job(l, k, T, src, out, out.numel() * out.element_size())
        tc = ref.codes.shape[0]
        gc = torch.full((max(tc * slot.r_eff, 1),), 0xEE, dtype=torch.uint8, device=DEV)
        gs = torch.full((max(tc * slot.n_act * 2, 1),), -1.0, dtype=torch.float32, device=DEV)
        dc.codec.unpack(djob, gc, gs, dc.ws, torch.cuda.current_stream())
        torch.cuda.synchronize()
        got_codes = gc.cpu().numpy()[: tc * slot.r_eff].reshape(tc, slot.r_eff)
        got_ss = gs.cpu().numpy()[: tc * slot.n_act * 2].reshape(tc, slot.n_act, 2)
        assert np.array_equal(got_codes, ref.codes)                      # T1 unpack
        assert np.array_equal(got_ss[:, :, 0].view(np.uint32), ref.shift.view(np.uint32))
        assert np.array_equal(got_ss[:, :, 1].view(np.uint32), ref.scale.view(np.uint32))


def test_edge_lengths_in_one_launch():
    """Empty, all-passthrough, one-row and ragged tensors share one launch."""
    wname, slots, _, _, calib = CASES["tiny"]
    w = synth.workload(wname)
    art = oracle_artifact(wname, slots, calib)
    op = art.params
    slot = art.slots[(0, 0)]
    dc = DevCodec(art.serialize())
    lens = [0, 1, 4, 60, 68, 69, 70, 131, 132, 133, 200, 1000]
    stores = [synth.storage(w, synth.gen_kv(w, 0, 0, synth.ROLE_EVAL, T, 7 + i))
              for i, T in enumerate(lens)]
    refs = [O.encode(s, op, slot, 0, 0) for s in stores]
    devs = [storage_to_dev(s) if s.shape[0] else torch.zeros((1, op.F), dtype=torch.float32, device=DEV)
            for s in stores]
    jobs, bufs = [], []
    for x, T in zip(devs, lens):
        n = dc.codec.encoded_bytes(0, 0, T)
        b = torch.full((n,), 0xEE, dtype=torch.uint8, device=DEV)
        bufs.append(b)
        jobs.append(K.make_job(0, 0, T, x, b, n))
    dc.codec.encode(jobs, dc.ws, torch.cuda.current_stream())
    assert np.all(dc.status(len(jobs)) == 0)
    for T, b, ref in zip(lens, bufs, refs):
        sb = bytes(b.cpu().numpy().tobytes())
        s1, w1, tc = O.split_rows(T, op.sink, op.window)
        rec0 = 64 + (s1 + w1) * op.F * op.elem_bytes
        assert sb[:rec0] == ref.stream[:rec0], T
        nbad, ntot, mx, _, _ = code_stats(sb, ref, op, slot, T)
        assert mx <= 1 and nbad <= max(1, ntot // 1000), (T, nbad)
    for od in (K.KVTC_F32, K.KVTC_BF16):
        outs, st = dc.decode([(0, 0, T, ref.stream) for T, ref in zip(lens, refs)], od, op.F)
        assert np.all(st == 0), st
        for T, out, ref in zip(lens, outs, refs):
            _decode_check(w, op, slot, ref.stream, T, out, od, 0, 0)
    # a launch with no compressed row at all still validates and copies
    short = [i for i, T in enumerate(lens) if T <= op.sink + op.window]
    for two in (False, True):
        outs, st = dc.decode([(0, 0, lens[i], refs[i].stream) for i in short], K.KVTC_F32, op.F,
                             two_stage=two)
        assert np.all(st == 0), st
        for i, out in zip(short, outs):
            _decode_check(w, op, slot, refs[i].stream, lens[i], out, K.KVTC_F32, 0, 0)
    # without compressed rows the two stages need no staging memory at all
    srcs = [to_dev_bytes(refs[i].stream, 16) for i in short]
    outs = [dc.out_buffer(lens[i], op.F, K.KVTC_F32) for i in short]
    jobs = [K.make_job(0, 0, lens[i], src, out, out.numel() * 4) for i, src, out in zip(short, srcs, outs)]
    assert dc.codec.staging_bytes(jobs) == 0
    s = torch.cuda.current_stream()
    dc.codec.decode_unpack(jobs, K.KVTC_F32, None, 0, dc.ws, s)
    dc.codec.decode_restore(jobs, K.KVTC_F32, None, 0, dc.ws, s)
    torch.cuda.synchronize()
    assert np.all(dc.status(len(jobs)) == 0)
    for i, out in zip(short, outs):
        _decode_check(w, op, slot, refs[i].stream, lens[i], out, K.KVTC_F32, 0, 0)


def _injected(F, G, widths, dtype, seed, s=4, w=16, mu_scale=1.0, lam=0.0):
    rng = np.random.default_rng(seed)
    widths = np.asarray(widths, np.uint8)
    r = int(np.count_nonzero(widths)) * G
    V = np.linalg.qr(rng.standard_normal((F, F)))[0][:, :r] if r else np.zeros((F, 0))
    p = O.Params(1, 1, F, s, w, G, 8, 16.0, dtype)
    sl = O.Slot(0, 0, F, G, widths, (mu_scale * rng.standard_normal(F)).astype(np.float32),
                np.full(F, lam), V.astype(np.float32))
    return p, sl


# Tokens x = mu + 3 z (z ~ N(0, 1)) around a mean of mu_ratio * 3 * N(0, 1)
# per feature, i.e. |mu| / spread = mu_ratio. With the slot's eigenvalues at
# the tokens' variance (9 per feature), mean09 sits just under the bound
# below which the encode folds the mean into the product (|mu|^2 <= sum of
# the eigenvalues); mean10 and mean100 are centred (their eigenvalues are
# given as zero, as are those of the other injected slots). Either way the
# code mismatches must stay within the bar.
MEAN_RATIOS = {"mean09": 0.9, "mean10": 10.0, "mean100": 100.0}


@pytest.mark.parametrize("variant", ["zero_bits", "reff256_g16", "reff256_g32", "odd_groups",
                                     "mean09", "mean10", "mean100"])
def test_injected_artifacts(variant):
    F = 1024
    if variant in MEAN_RATIOS:
        wd = np.zeros(64, np.uint8)
        wd[:6] = [8, 8, 7, 7, 6, 4]
        p, sl = _injected(F, 16, wd, O.DTYPE_BF16, 5, mu_scale=3.0 * MEAN_RATIOS[variant],
                          lam=9.0 if variant == "mean09" else 0.0)
    elif variant == "zero_bits":
        p, sl = _injected(F, 16, np.zeros(64), O.DTYPE_BF16, 1)
    elif variant == "reff256_g16":
        wd = np.zeros(64, np.uint8)
        wd[:16] = [8, 1, 7, 2, 6, 3, 5, 4, 8, 8, 1, 1, 3, 3, 6, 2]
        p, sl = _injected(F, 16, wd, O.DTYPE_BF16, 2)
    elif variant == "reff256_g32":
        wd = np.zeros(32, np.uint8)
        wd[:8] = [8, 7, 6, 5, 4, 3, 2, 1]
        p, sl = _injected(F, 32, wd, O.DTYPE_BF16, 3)
    else:
        wd = np.zeros(64, np.uint8)
        wd[[0, 3, 9, 40, 63]] = [5, 8, 1, 2, 3]    # odd n_act, scattered groups
        p, sl = _injected(F, 16, wd, O.DTYPE_BF16, 4)
    art = O.Artifact(p, {(0, 0): sl})
    dc = DevCodec(art.serialize())
    assert dc.codec.slot(0, 0).folded_mean == (1 if variant == "mean09" else 0)
    rng = np.random.default_rng(9)
    T = 777
    x = (rng.standard_normal((T, F)) * 3).astype(np.float32)
    if variant in MEAN_RATIOS:
        x = (x + sl.mu32).astype(np.float32)
    store = O.f32_to_bf16_bits(x)
    ref = O.encode(store, p, sl, 0, 0)
    sb = dc.encode([(0, 0, storage_to_dev(store))])[0]
    s1, w1, tc = O.split_rows(T, p.sink, p.window)
    rec0 = 64 + (s1 + w1) * F * 2
    assert sb[:rec0] == ref.stream[:rec0]
    # T1: the oracle's codes and (shift, scale) pack to the oracle's stream
    n = dc.codec.encoded_bytes(0, 0, T)
    buf = torch.zeros(n, dtype=torch.uint8, device=DEV)
    codes = torch.from_numpy(np.ascontiguousarray(ref.codes)).to(DEV)
    ss = torch.from_numpy(np.ascontiguousarray(np.stack([ref.shift, ref.scale], axis=2))).to(DEV)
    dc.codec.pack(K.make_job(0, 0, T, storage_to_dev(store), buf, n), codes, ss, dc.ws,
                  torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert bytes(buf.cpu().numpy().tobytes()) == ref.stream
    nbad, ntot, mx, _, _ = code_stats(sb, ref, p, sl, T)
    print(f"{variant}: code mismatches {nbad}/{ntot}, max step {mx}")
    assert mx <= 1 and nbad <= max(2, ntot * CODE_RATE), (nbad, ntot)
    for od in (K.KVTC_F32, K.KVTC_BF16):
        for two in (False, True):
            # staging that stage 1 leaves unwritten holds NaN bit patterns
            outs, st = dc.decode([(0, 0, T, ref.stream)], od, F, two_stage=two, stg_fill=0xFF)
            assert np.all(st == 0)
            _decode_check(None, p, sl, ref.stream, T, outs[0], od, 0, 0)


# (F, G, widths per group): every width 1..8 with both group sizes, and
# scattered active groups of mixed widths (odd n_act, dropped groups between).
IDENTITY_CASES = {f"w{b}_g{G}": (4 * G, G, [b] * 4) for b in range(1, 9) for G in (16, 32)}
IDENTITY_CASES["mixed_g16"] = (512, 16, [5, 0, 0, 8, 0, 1, 2, 0, 0, 3, 7] + [0] * 20 + [4])
IDENTITY_CASES["mixed_g32"] = (512, 32, [0, 6, 0, 1, 8, 0, 3, 0, 0, 0, 2, 0, 0, 0, 0, 5])


def _grid_tokens(widths, G, T, rng):
    """Tokens whose every active group lies on its own width's grid:
    (m + q) 2^e with q in [0, 2^b - 1] (0 and 2^b - 1 both present), |m + q|
    <= 255 (bfloat16-exact), e in [-6, 2] per (token, group); zero elsewhere."""
    F = G * len(widths)
    x = np.zeros((T, F), np.float32)
    for g, b in enumerate(int(v) for v in widths):
        if not b:
            continue
        k = 2 ** b - 1
        e = rng.integers(-6, 3, T).astype(np.float64)
        m = rng.integers(-k, 256 - k, T)
        q = rng.integers(0, k + 1, (T, G))
        q[:, 0], q[:, G // 2 + 1] = 0, k
        x[:, g * G:(g + 1) * G] = (m[:, None] + q) * 2.0 ** e[:, None]
    return x


def test_mixed_record_sizes_in_one_launch():
    """Two slots with the same K-step count (six 16-component groups) but
    record sizes 128 bytes (a multiple of 16: LDS rows padded to 144) and
    142 bytes decoded in one launch, through both decode routes: every job's
    record rows must fit the batch's LDS rows."""
    F, G, T = 1024, 16, 901
    rng = np.random.default_rng(21)
    V = np.linalg.qr(rng.standard_normal((F, F)))[0]
    slots = {}
    for kind, wd6 in ((0, [8, 8, 8, 8, 4, 4]), (1, [8, 8, 8, 8, 8, 7])):
        wd = np.zeros(F // G, np.uint8)
        wd[:6] = wd6
        slots[(0, kind)] = O.Slot(0, kind, F, G, wd, rng.standard_normal(F).astype(np.float32),
                                  np.zeros(F), V[:, :96].astype(np.float32))
    assert [sl.record_bytes for sl in slots.values()] == [128, 142]
    p = O.Params(1, 1, F, 4, 16, G, 8, 16.0, O.DTYPE_BF16)
    dc = DevCodec(O.Artifact(p, slots).serialize())
    items = []
    for rep in range(3):
        for kind in (0, 1):
            x = (rng.standard_normal((T, F)) * 2).astype(np.float32)
            ref = O.encode(O.f32_to_bf16_bits(x), p, slots[(0, kind)], 0, kind)
            items.append((kind, ref))
    for two in (False, True):
        outs, st = dc.decode([(0, kind, T, ref.stream) for kind, ref in items], K.KVTC_F32, F, two_stage=two)
        assert np.all(st == 0), st
        for (kind, ref), out in zip(items, outs):
            _decode_check(None, p, slots[(0, kind)], ref.stream, T, out, K.KVTC_F32, 0, kind)


def test_folded_and_centred_slots_in_one_call():
    """One kvtc_encode call over jobs of a slot that folds the mean (mean just
    under its spread) and of one that centres it (mean ten spreads), in
    alternation: the host puts each product form in launches of its own,
    and every stream must match the oracle's header, passthrough rows and
    codes."""
    F = 1024
    wd = np.zeros(64, np.uint8)
    wd[:6] = [8, 8, 7, 7, 6, 4]
    p, sf = _injected(F, 16, wd, O.DTYPE_BF16, 5, mu_scale=3.0 * 0.9, lam=9.0)
    _, s0 = _injected(F, 16, wd, O.DTYPE_BF16, 6, mu_scale=3.0 * 10.0)
    sc = O.Slot(0, 1, F, 16, s0.widths, s0.mu32, s0.lam, s0.V32)
    dc = DevCodec(O.Artifact(p, {(0, 0): sf, (0, 1): sc}).serialize())
    assert dc.codec.slot(0, 0).folded_mean == 1 and dc.codec.slot(0, 1).folded_mean == 0
    rng = np.random.default_rng(13)
    items, refs = [], []
    for kind, sl, T in ((0, sf, 777), (1, sc, 1300), (0, sf, 64), (1, sc, 2049), (0, sf, 3000)):
        x = (rng.standard_normal((T, F)) * 3 + sl.mu32).astype(np.float32)
        store = O.f32_to_bf16_bits(x)
        refs.append((O.encode(store, p, sl, 0, kind), sl, T))
        items.append((0, kind, storage_to_dev(store)))
    for sb, (ref, sl, T) in zip(dc.encode(items), refs):
        s1, w1, _ = O.split_rows(T, p.sink, p.window)
        rec0 = 64 + (s1 + w1) * F * 2
        assert sb[:rec0] == ref.stream[:rec0]
        nbad, ntot, mx, _, _ = code_stats(sb, ref, p, sl, T)
        assert mx <= 1 and nbad <= max(2, ntot * CODE_RATE), (T, nbad, ntot)


@pytest.mark.parametrize("dtype", [O.DTYPE_BF16, O.DTYPE_F32])
@pytest.mark.parametrize("case", list(IDENTITY_CASES))
def test_identity_basis_is_exact(case, dtype):
    """mu = 0, V = identity on the active groups, tokens on each group's grid:
    the production encode's stream equals the oracle's byte for byte (every
    code, shift, scale and record bit), and the production decode (both
    routes) returns the input exactly, in both output types."""
    F, G, widths = IDENTITY_CASES[case]
    T = 300
    rng = np.random.default_rng(8)
    widths = np.asarray(widths, np.uint8)
    act = np.concatenate([np.arange(g * G, (g + 1) * G) for g in np.nonzero(widths)[0]])
    p = O.Params(1, 1, F, 2, 3, G, 8, 12.0, dtype)
    sl = O.Slot(0, 0, F, G, widths, np.zeros(F, np.float32), np.zeros(F),
                np.eye(F, dtype=np.float32)[:, act])
    x = _grid_tokens(widths, G, T, rng)
    store = O.f32_to_bf16_bits(x) if dtype == O.DTYPE_BF16 else x
    ref = O.encode(store, p, sl, 0, 0)
    dc = DevCodec(O.Artifact(p, {(0, 0): sl}).serialize())
    sb = dc.encode([(0, 0, storage_to_dev(store))])[0]
    assert sb == ref.stream
    for od in (K.KVTC_F32, K.KVTC_BF16):
        for two in (False, True):
            outs, st = dc.decode([(0, 0, T, ref.stream)], od, F, two_stage=two)
            assert np.all(st == 0)
            got = outs[0].cpu().numpy()
            want = x if od == K.KVTC_F32 else O.f32_to_bf16_bits(x).view(np.int16)
            assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), (od, two)


def test_corrupt_stream_is_rejected_without_writes():
    wname, slots, T, _, calib = CASES["tiny"]
    w = synth.workload(wname)
    art = oracle_artifact(wname, slots, calib)
    op = art.params
    slot = art.slots[(0, 0)]
    dc = DevCodec(art.serialize())
    store = synth.storage(w, synth.gen_kv(w, 0, 0, synth.ROLE_EVAL, T))
    ref = O.encode(store, op, slot, 0, 0)
    for off, want in ((0, K.KVTC_E_CORRUPT), (4, K.KVTC_E_CORRUPT), (12, K.KVTC_E_MISMATCH),
                      (34, K.KVTC_E_MISMATCH), (41, K.KVTC_E_MISMATCH)):
        bad = bytearray(ref.stream)
        bad[off] ^= 0x21
        for two in (False, True):
            outs, st = dc.decode([(0, 0, T, bytes(bad))], K.KVTC_F32, op.F, two_stage=two)
            assert st[0] == want, (off, st)
            assert torch.all(outs[0] == -7.0), "a rejected stream wrote output rows"


def test_bad_block_table_entry_is_reported():
    wname, slots, T, _, calib = CASES["tiny"]
    w = synth.workload(wname)
    art = oracle_artifact(wname, slots, calib)
    op = art.params
    dc = DevCodec(art.serialize())
    store = synth.storage(w, synth.gen_kv(w, 0, 0, synth.ROLE_EVAL, T))
    ref = O.encode(store, op, art.slots[(0, 0)], 0, 0)
    nblk = T // 16
    table = np.arange(nblk, dtype=np.int32)
    table[5] = nblk + 3                            # out of range
    bt = torch.from_numpy(table).to(DEV)
    outs, st = dc.decode([(0, 0, T, ref.stream)], K.KVTC_F32, op.F, [(bt, 16, nblk)])
    assert st[0] == K.KVTC_E_INVALID
    got = outs[0].cpu().numpy()
    full, _ = O.decode(ref.stream, op, art.slots[(0, 0)], 0, 0, T)
    ok_rows = np.r_[0:80, 96:T]                    # block 5 = tokens 80..95 is skipped
    M = np.abs(full).max()
    assert np.abs(got[ok_rows] - full[ok_rows]).max() / M <= DEC_TOL


def test_full_size_launch_llama8b():
    """The benchmark's launch shape: 64 tensors of 8192 tokens in one call
    (jobs over 4 calibrated slots, 16 tensors each); every output compared."""
    wname, slots, T, _, calib = CASES["llama31_8b"]
    w = synth.workload(wname)
    art = oracle_artifact(wname, slots, calib)
    op = art.params
    dc = DevCodec(art.serialize())
    srcs = {}
    for (l, k) in slots:
        store = synth.storage(w, synth.gen_kv(w, l, k, synth.ROLE_EVAL, T, 5))
        srcs[(l, k)] = (store, storage_to_dev(store), O.encode(store, op, art.slots[(l, k)], l, k))
    order = [slots[i % 4] for i in range(64)]
    streams = dc.encode([(l, k, srcs[(l, k)][1]) for l, k in order])
    bad = total = worst = 0
    for (l, k), sb in zip(order, streams):
        ref = srcs[(l, k)][2]
        nb, nt, mx, _, _ = code_stats(sb, ref, op, art.slots[(l, k)], T)
        assert sb[:64] == ref.stream[:64]
        bad, total, worst = bad + nb, total + nt, max(worst, mx)
    assert worst <= 1 and bad / total <= CODE_RATE, (bad, total)
    outs, st = dc.decode([(l, k, T, srcs[(l, k)][2].stream) for l, k in order], K.KVTC_BF16, op.F)
    assert np.all(st == 0)
    refs = {key: O.decode(v[2].stream, op, art.slots[key], key[0], key[1], T)[0]
            for key, v in srcs.items()}
    for (l, k), out in zip(order, outs):
        full = refs[(l, k)]
        g = bf16_out_to_f64(out[:T])
        M = np.abs(full).max()
        assert np.all(np.abs(g - full) <= DEC_TOL * M + 2.0 ** -8 * np.abs(full))


def test_two_stream_layer_pipeline_matches_fused():
    """Layer-by-layer decode on two streams over 4 layers x {K, V} x 2
    requests of the Qwen2.5-7B shape: stage 1 of layer l+1 overlaps stage 2
    of layer l, two staging buffers and workspaces alternate, and from layer 2
    on stage 1 waits until stage 2 of layer l-2 has released its buffer. The
    paged pool equals the fused decode's bit for bit and the oracle's within
    the decode tolerance."""
    wname = "qwen25_7b_paged"
    w = synth.workload(wname)
    T, reqs = 8192, 2
    slots = [(l, k) for l in range(4) for k in (0, 1)]
    art = oracle_artifact(wname, slots, 4096)
    op = art.params
    items = []
    for (l, k) in slots:
        for r in range(reqs):
            store = synth.storage(w, synth.gen_kv(w, l, k, synth.ROLE_EVAL, T, r))
            items.append((l, k, O.encode(store, op, art.slots[(l, k)], l, k)))
    dc = DevCodec(art.serialize())
    bs = w.block_size
    per_req = (T + bs - 1) // bs
    rng = np.random.default_rng(5)
    layers = sorted({l for l, _, _ in items})
    pool_blocks = per_req * len(items)
    perm = rng.permutation(pool_blocks).astype(np.int32)
    srcs, tables = [], []
    for i, (l, k, ref) in enumerate(items):
        srcs.append(to_dev_bytes(ref.stream, 16))
        tables.append(perm[i * per_req:(i + 1) * per_req].copy())
    dtables = [torch.from_numpy(t).to(DEV) for t in tables]
    pool_f = torch.full((pool_blocks * bs, op.F), -7, dtype=torch.int16, device=DEV)
    pool_p = torch.full_like(pool_f, -7)
    nbytes = pool_f.numel() * 2
    fused_jobs, pipe_jobs = [], {l: [] for l in layers}
    for i, (l, k, ref) in enumerate(items):
        fused_jobs.append(K.make_job(l, k, T, srcs[i], pool_f, nbytes, dtables[i], bs, pool_blocks))
        pipe_jobs[l].append(K.make_job(l, k, T, srcs[i], pool_p, nbytes, dtables[i], bs, pool_blocks))
    s = torch.cuda.current_stream()
    assert np.all(dc.decode_jobs(fused_jobs, K.KVTC_BF16) == 0)
    nst = max(dc.codec.staging_bytes(js) for js in pipe_jobs.values())
    stg = [torch.full((nst,), 0xFF, dtype=torch.uint8, device=DEV) for _ in range(2)]
    nws = max(K.kvtc_workspace_bytes(len(js)) for js in pipe_jobs.values())
    wss = [torch.zeros(nws // 4, dtype=torch.int32, device=DEV) for _ in range(2)]
    su, sr = torch.cuda.Stream(), torch.cuda.Stream()
    ev_u = [torch.cuda.Event() for _ in layers]
    ev_r = [torch.cuda.Event() for _ in layers]
    start = torch.cuda.Event()
    start.record(s)
    su.wait_event(start)
    sr.wait_event(start)
    status = []
    for idx, l in enumerate(layers):
        b = idx % 2
        if idx >= 2:
            su.wait_event(ev_r[idx - 2])      # buffer b is free once layer idx-2 is restored
        dc.codec.decode_unpack(pipe_jobs[l], K.KVTC_BF16, stg[b], nst, wss[b], su)
        ev_u[idx].record(su)
        sr.wait_event(ev_u[idx])
        dc.codec.decode_restore(pipe_jobs[l], K.KVTC_BF16, stg[b], nst, wss[b], sr)
        ev_r[idx].record(sr)
        if idx >= len(layers) - 2:            # the last use of each workspace
            status.append((b, len(pipe_jobs[l])))
    torch.cuda.synchronize()
    for b, n in status:
        assert np.all(K.kvtc_read_device_status(wss[b], n, s) == 0)
    assert torch.equal(pool_f, pool_p)
    assert not torch.any(pool_f == -7)   # every block of the pool was written
    t = np.arange(T)
    for i, (l, k, ref) in enumerate(items):
        rows = torch.from_numpy(tables[i][t // bs] * bs + t % bs).to(DEV)
        _decode_check(w, op, art.slots[(l, k)], ref.stream, T, pool_p, K.KVTC_BF16, l, k, rows)
