"""Checks that pin the CPU oracle to facts fixed outside itself.

Each check raises AssertionError on failure.  They are collected as tests in
test_oracle_pins.py and re-run against deliberately broken copies of the oracle
in test_oracle_mutations.py, which shows that a plausible mistake anywhere in
the oracle fails at least one of them.

Sources of truth used here, none of which is the oracle's own arithmetic:
  * hand-worked fixtures in tests/golden/ (each cites the page section);
  * independent library routines: torch's bfloat16 rounding, numpy.linalg.eigh
    of the covariance (the oracle uses an SVD of the data), exact rational
    arithmetic (fractions) for dot products;
  * closed forms: Parseval for an orthonormal basis, the uniform quantizer's
    half-step bound, exact reconstruction on a dyadic grid with an exactly
    orthonormal Hadamard basis;
  * brute force over every width vector for a few groups;
  * the KV size the page states for Llama 3.1 8B (128 MiB per 1K tokens).
"""
from __future__ import annotations

import fractions
import itertools
import json
import os
import struct

import numpy as np

import oracle.kvtc_lossless as LZ
import oracle.kvtc_oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------- helpers ---

def small_params(F=64, G=16, bpv=4.0, s=4, w=8, dtype=O.DTYPE_F32, max_bits=8):
    return O.Params(1, 1, F, s, w, G, max_bits, bpv, dtype)


def hadamard(n):
    h = np.array([[1.0]])
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def injected_slot(V32, widths, mu32, G):
    F = V32.shape[0]
    return O.Slot(0, 0, F, G, np.asarray(widths, np.uint8), np.asarray(mu32, np.float32),
                  np.zeros(F), np.asarray(V32, np.float32))


def family_b_small(seed=7, n=4096):
    """A small family-B-like tensor: 2 heads x 32 dims sharing a rank-12 latent."""
    rng = np.random.default_rng(seed)
    d, r, H = 32, 12, 2
    U, _ = np.linalg.qr(rng.standard_normal((d, r)))
    M = np.concatenate([np.linalg.qr(rng.standard_normal((d, d)))[0] @ U for _ in range(H)])
    sig = np.arange(1, r + 1) ** -1.2 * 4.0
    mean = rng.standard_normal(d * H)
    x = (rng.standard_normal((n, r)) * sig) @ M.T + mean + 1e-3 * rng.standard_normal((n, d * H))
    return x.astype(np.float32), M


def brute_force_widths(D, G, budget):
    """Enumerate every width vector and order them by (objective, bits,
    lexicographically largest widths).  D must hold exact binary fractions
    small enough that every sum is exact in fp64, so no summation order
    matters."""
    n_g, nb = D.shape
    ws = np.array(list(itertools.product(range(nb), repeat=n_g)), np.int64)
    cost = np.sum(G * ws + 64 * (ws > 0), axis=1)
    obj = np.sum(D[np.arange(n_g), ws], axis=1)
    ok = cost <= budget
    ws, cost, obj = ws[ok], cost[ok], obj[ok]
    # lexsort: last key is primary
    keys = [-ws[:, g] for g in range(n_g - 1, -1, -1)] + [cost, obj]
    i = np.lexsort(keys)[0]
    return ws[i].astype(np.uint8), obj[i]


def brute_force_global(Ds, G, budget, cap):
    """Every width vector of every tensor at once (equal group counts), kept
    if each tensor has at most cap active groups and the bits sum to at most
    len(Ds) * budget, ordered by (objective, total bits, most bits to earlier
    tensors, lexicographically largest widths).  D values must be exact
    binary fractions so no summation order matters."""
    S, (n_g, nb) = len(Ds), Ds[0].shape
    ws = np.array(list(itertools.product(range(nb), repeat=S * n_g)), np.int64).reshape(-1, S, n_g)
    bits = np.sum(G * ws + 64 * (ws > 0), axis=2)                    # [N, S]
    obj = sum(np.sum(Ds[s][np.arange(n_g), ws[:, s]], axis=1) for s in range(S))
    ok = (np.sum(bits, axis=1) <= S * budget) & np.all(np.sum(ws > 0, axis=2) <= cap, axis=1)
    ws, bits, obj = ws[ok], bits[ok], obj[ok]
    flat = ws.reshape(len(ws), -1)
    keys = ([-flat[:, i] for i in range(S * n_g - 1, -1, -1)]
            + [-bits[:, s] for s in range(S - 1, -1, -1)] + [np.sum(bits, axis=1), obj])
    i = np.lexsort(keys)[0]
    return [ws[i, s].astype(np.uint8) for s in range(S)], obj[i]


def three_scaled_tensors():
    """Three family-B-like tensors of very different energy (scales 1, 4, 1/4)."""
    x, _ = family_b_small(seed=12, n=1500)
    y, _ = family_b_small(seed=13, n=1500)
    z, _ = family_b_small(seed=14, n=1500)
    return [(0, 0, x), (1, 0, 4 * y), (0, 1, z / 4)]


# ------------------------------------------------------------------- pins ---

def check_bf16_vs_torch():
    import torch
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 10.0 ** rng.integers(-6, 6, 20000),
        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -130, 0.0, -0.0,
                  3.0e38, 1.0 - 2 ** -24], np.float32)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = O.bf16_rne(x)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), "bf16 rounding differs from torch"


def check_fnv_vectors():
    # Published FNV-1a 64-bit test vectors.
    assert O.fnv1a64(b"") == 0xCBF29CE484222325
    assert O.fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert O.fnv1a64(b"foobar") == 0x85944171F73967E8


def check_pack_golden():
    for case in golden("pack_examples.json")["cases"]:
        q = np.array([case["codes"]], np.uint8)
        got = O.pack_codes(q, case["b"]).tobytes().hex()
        assert got == case["bytes_hex"], (case["b"], got, case["bytes_hex"])
        back = O.unpack_codes(np.frombuffer(bytes.fromhex(case["bytes_hex"]), np.uint8)[None, :],
                              16, case["b"])
        assert np.array_equal(back, q), case["b"]


def check_pack_roundtrip():
    rng = np.random.default_rng(1)
    for G in (16, 32):
        for b in range(1, 9):
            q = rng.integers(0, 2 ** b, (37, G)).astype(np.uint8)
            p = O.pack_codes(q, b)
            assert p.shape == (37, G * b // 8)
            assert np.array_equal(O.unpack_codes(p, G, b), q)


def check_quantizer_golden():
    for case in golden("quantizer_examples.json")["cases"]:
        c = np.array([case["c"]], np.float32)
        q, shift, scale = O.quantize_fp32(c, case["b"])
        assert q.tolist()[0] == case["q"], (case, q)
        assert float(shift[0]) == case["shift"] and float(scale[0]) == case["scale"]


def check_quantizer_bound():
    rng = np.random.default_rng(2)
    for b in range(1, 9):
        c = (rng.standard_normal((500, 16)) * 10.0 ** rng.uniform(-3, 3, (500, 1))).astype(np.float32)
        q, shift, scale = O.quantize_fp32(c, b)
        k = 2 ** b - 1
        assert q.max() <= k
        assert np.all(q.min(axis=1) == 0) and np.all(q.max(axis=1) == k)
        chat = O.dequantize(q, shift, scale, b)
        step = scale.astype(np.float64) / k
        err = np.abs(chat - c.astype(np.float64))
        assert np.all(err <= step[:, None] * (0.5 + 1e-5) + 1e-6 * np.abs(c)), b


def check_pca_invariants():
    x, M = family_b_small()
    p = O.Params(1, 2, 32, 4, 8, 16, 8, 2.0, O.DTYPE_F32)
    sl = O.calibrate(x, p, 0, 0)
    V, lam = sl.V64, sl.lam
    F = V.shape[0]
    assert np.allclose(V.T @ V, np.eye(F), atol=1e-10), "basis not orthonormal"
    rows = x[4:-8].astype(np.float64)
    xc = rows - rows.mean(axis=0)
    cov = xc.T @ xc / xc.shape[0]
    proj = V.T @ cov @ V
    off = proj - np.diag(np.diag(proj))
    assert np.abs(off).max() <= 1e-9 * np.abs(proj).max(), "projected covariance not diagonal"
    assert np.allclose(np.diag(proj), lam, rtol=1e-9, atol=1e-12)
    ev = np.linalg.eigh(cov)[0][::-1]                    # independent route
    assert np.allclose(lam, ev, rtol=1e-8, atol=1e-12 * ev[0]), "eigenvalues disagree with eigh"
    assert np.all(np.diff(lam) <= 0), "components not sorted by variance"
    for j in range(F):
        i = int(np.argmax(np.abs(V[:, j])))
        assert V[i, j] > 0, "sign rule"
    # the planted rank-12 subspace is recovered (principal angles ~ 0)
    Q = np.linalg.qr(M)[0]
    s = np.linalg.svd(Q.T @ V[:, :12], compute_uv=False)
    assert s.min() > 0.999, s.min()
    # mean is the mean of the rows [s, n - w)
    assert np.allclose(sl.mu64, rows.mean(axis=0), rtol=0, atol=1e-12)


def check_parseval():
    x, _ = family_b_small(seed=3, n=2048)
    p = O.Params(1, 2, 32, 4, 8, 16, 8, 2.0, O.DTYPE_F32)
    sl = O.calibrate(x, p, 0, 0)
    rows = x[4:-8].astype(np.float64)
    xc = rows - rows.mean(axis=0)
    feat = np.mean(np.sum(xc * xc, axis=1))
    assert np.isclose(np.sum(sl.D[:, 0]), feat, rtol=1e-10), "Parseval"
    # the retained error in feature space equals the table's prediction
    C = xc @ sl.V64
    xhat = np.zeros_like(xc)
    for g in range(sl.D.shape[0]):
        b = int(sl.widths[g])
        cols = slice(16 * g, 16 * g + 16)
        if b:
            xhat += O.quant_dequant_fp64(C[:, cols], b) @ sl.V64[:, cols].T
    err = np.mean(np.sum((xc - xhat) ** 2, axis=1))
    pred = sum(sl.D[g, int(sl.widths[g])] for g in range(sl.D.shape[0]))
    assert np.isclose(err, pred, rtol=1e-9), "distortion table does not predict the error"


def check_distortion_bound():
    x, _ = family_b_small(seed=4, n=1024)
    p = O.Params(1, 2, 32, 4, 8, 16, 8, 2.0, O.DTYPE_F32)
    sl = O.calibrate(x, p, 0, 0)
    rows = x[4:-8].astype(np.float64)
    C = (rows - rows.mean(axis=0)) @ sl.V64
    for g in range(sl.D.shape[0]):
        cg = C[:, 16 * g:16 * g + 16]
        rng_ = cg.max(axis=1) - cg.min(axis=1)
        for b in range(1, 9):
            bound = np.mean(16 * (rng_ / (2 ** b - 1) / 2) ** 2)
            assert sl.D[g, b] <= bound * (1 + 1e-9)
        assert np.isclose(sl.D[g, 0], np.mean(np.sum(cg * cg, axis=1)))


def check_dp_golden():
    gd = golden("dp_examples.json")
    D = np.array(gd["D"])
    for case in gd["cases"]:
        w = O.dp_allocate(D, gd["G"], case["budget"])
        assert w.tolist() == case["widths"], (case, w)
        assert sum(D[g, b] for g, b in enumerate(w)) == case["objective"]


def check_dp_bruteforce():
    rng = np.random.default_rng(5)
    for trial in range(40):
        n_g = int(rng.integers(1, 5))
        G = int(rng.choice([16, 32]))
        e = np.sort(rng.uniform(0, 100, n_g))[::-1]
        # realistic tables: decreasing in b, exact small dyadic values so ties are real
        D = np.array([[np.round(e[g] * 4.0 ** -b * 64) / 64 for b in range(9)] for g in range(n_g)])
        if trial % 5 == 0:
            D[-1] = 0.0
        for budget in (0, 63, 80, 100, 150, 300, 500, 900):
            w = O.dp_allocate(D, G, budget)
            bw, bobj = brute_force_widths(D, G, budget)
            assert np.array_equal(w, bw), (D, G, budget, w, bw)
    # optimum non-increasing in the budget
    D = np.array([[50 * 3.0 ** -b for b in range(9)], [20 * 3.0 ** -b for b in range(9)],
                  [5 * 3.0 ** -b for b in range(9)]])
    prev = np.inf
    for budget in range(0, 700, 16):
        w = O.dp_allocate(D, 16, budget)
        obj = sum(D[g, b] for g, b in enumerate(w))
        assert obj <= prev + 1e-12
        assert sum(16 * int(b) + (64 if b else 0) for b in w) <= budget
        prev = obj


def check_dp_global_bruteforce():
    """The global allocation (several tensors, one budget, a cap on active
    groups per tensor) against brute force, ties included."""
    rng = np.random.default_rng(11)
    for trial in range(24):
        S = int(rng.integers(1, 4))
        n_g = 1 if S == 3 else int(rng.integers(1, 3))
        nb = int(rng.integers(2, 5))
        G = int(rng.choice([8, 16]))
        Ds = []
        for _ in range(S):
            e = np.sort(rng.uniform(0, 50, n_g))[::-1]
            Ds.append(np.array([[np.round(e[g] * 4.0 ** -b * 64) / 64 for b in range(nb)]
                                for g in range(n_g)]))
        if trial % 4 == 1 and S > 1:
            Ds[1] = Ds[0].copy()                # identical tensors: a tie between tensors
        if trial % 6 == 2:
            Ds[-1][:] = 0.0
        for budget in (0, 60, 72, 100, 180):
            for cap in (0, 1, 2):
                ws = O.dp_allocate_global(Ds, G, budget, cap)
                bw, _ = brute_force_global(Ds, G, budget, cap)
                assert all(np.array_equal(a, b) for a, b in zip(ws, bw)), (trial, budget, cap, ws, bw)
    # one tensor and no binding cap: the per-tensor DP
    gd = golden("dp_examples.json")
    D = np.array(gd["D"])
    for case in gd["cases"]:
        (w,) = O.dp_allocate_global([D], gd["G"], case["budget"], D.shape[0])
        assert w.tolist() == case["widths"], (case, w)


def check_global_budget_moves_bits():
    """One budget over three tensors of very different energy: never worse
    than a budget per tensor, strictly better here, within the total bits
    and the cap."""
    p = small_params(F=64, G=16, bpv=2.0)
    ins = three_scaled_tensors()
    per = O.calibrate_set(ins, p)
    glob = O.calibrate_set(ins, p, global_budget=True, max_active=2)
    obj = lambda sl: sum(sl.D[g, b] for g, b in enumerate(sl.widths))
    bits = lambda sl: sum(16 * int(b) + (64 if b else 0) for b in sl.widths)
    o_per = sum(obj(sl) for sl in per.values())
    o_glob = sum(obj(sl) for sl in glob.values())
    assert o_glob < 0.9 * o_per, (o_glob, o_per)
    assert sum(bits(sl) for sl in glob.values()) <= 3 * p.budget_bits
    assert all(sl.n_act <= 2 for sl in glob.values())
    big = glob[(1, 0)]
    assert bits(big) > p.budget_bits and bits(glob[(0, 1)]) < p.budget_bits
    for k, sl in per.items():                 # without the flag: calibrate() per tensor
        ref = O.calibrate(ins[[i[:2] for i in ins].index(k)][2], p, *k)
        assert np.array_equal(sl.widths, ref.widths) and np.array_equal(sl.V32, ref.V32)


def check_shared_basis():
    """A basis shared by the tensors of one kind: a single tensor gives
    calibrate()'s slot; a copy of a tensor shifted by a constant row gives
    the same basis and its own mean; for different tensors the eigenvalues
    are those of the summed scatter matrices (numpy eigh); K and V are never
    pooled together."""
    p = small_params(F=64, G=16, bpv=2.0)
    x, _ = family_b_small(seed=4, n=1500)
    one = O.calibrate_set([(0, 0, x)], p, shared_basis=True)[(0, 0)]
    ref = O.calibrate(x, p, 0, 0)
    assert np.array_equal(one.V32, ref.V32) and np.array_equal(one.mu32, ref.mu32)
    off = np.round(np.random.default_rng(2).standard_normal(64) * 8) * 0.5
    x2 = x.astype(np.float64) + off
    pair = O.calibrate_set([(0, 0, x), (1, 0, x2)], p, shared_basis=True)
    k = 12                                    # the planted rank; the gap after it is huge
    for sl in pair.values():
        Pa, Pb = sl.V64[:, :k] @ sl.V64[:, :k].T, ref.V64[:, :k] @ ref.V64[:, :k].T
        assert np.abs(Pa - Pb).max() < 1e-8
        assert np.allclose(sl.lam[:k], ref.lam[:k], rtol=1e-9)
    assert np.array_equal(pair[(1, 0)].mu32, O.calibrate(x2, p, 1, 0).mu32)
    y, _ = family_b_small(seed=9, n=1200)
    z, _ = family_b_small(seed=10, n=1000)
    mix = O.calibrate_set([(0, 0, x), (1, 0, y), (0, 1, z)], p, shared_basis=True)
    rows = [r[p.sink: len(r) - p.window].astype(np.float64) for r in (x, y)]
    scat = sum((r - r.mean(axis=0)).T @ (r - r.mean(axis=0)) for r in rows)
    ev = np.linalg.eigvalsh(scat / sum(len(r) for r in rows))[::-1]
    for key in ((0, 0), (1, 0)):
        assert np.allclose(mix[key].lam[:24], ev[:24], rtol=1e-8, atol=1e-12 * ev[0])
    assert np.array_equal(mix[(0, 0)].V32, mix[(1, 0)].V32)
    assert np.array_equal(mix[(0, 1)].V32, O.calibrate(z, p, 0, 1).V32)


def lossless_streams():
    """KVTC streams of several shapes for the lossless stage: family-B data in
    bf16 and f32 at G = 16 and 32, every width 1..8 on an injected slot, no
    active group, and the short lengths (0, 1, all passthrough, one
    compressed row, a ragged last chunk)."""
    rng = np.random.default_rng(31)
    out = []
    x, _ = family_b_small(seed=17, n=2600)
    for G, dt in ((16, O.DTYPE_BF16), (32, O.DTYPE_F32)):
        p = small_params(F=64, G=G, bpv=3.0, dtype=dt)
        sl = O.calibrate(x[:2000], p, 0, 0)
        xs = O.f32_to_bf16_bits(x[2000:]) if dt == O.DTYPE_BF16 else x[2000:]
        for T in (600, 0, 1, 12, 13):
            out.append((p, sl, T, O.encode(xs[:T], p, sl, 0, 0).stream))
    p = small_params(F=128, G=16, bpv=12.0, dtype=O.DTYPE_BF16)
    sl = injected_slot(np.eye(128), [1, 2, 3, 4, 5, 6, 7, 8], np.zeros(128), 16)
    xs = O.f32_to_bf16_bits(rng.standard_normal((1100, 128)).astype(np.float32))
    out.append((p, sl, 1100, O.encode(xs, p, sl, 0, 0).stream))
    sl0 = injected_slot(np.zeros((128, 0)), [0] * 8, np.zeros(128), 16)
    out.append((p, sl0, 300, O.encode(xs[:300], p, sl0, 0, 0).stream))
    # a width per component (reading L1c): widths 0..8 mixed inside every
    # active group, so chunks end in padding bits and some codes are empty
    p = small_params(F=64, G=16, bpv=3.0, dtype=O.DTYPE_BF16)
    pc = O.calibrate_set([(0, 0, x[:2000])], p, component_widths=True)[(0, 0)]
    cw = pc.cwidths.copy()
    for a, g in enumerate(pc.active_groups):
        cw[g * 16:(g + 1) * 16] = [(3 * a + 5 * i + 1) % 9 for i in range(16)]
        cw[g * 16] = max(cw[g * 16], 1)
    pc.cwidths = cw
    pc.widths = cw.reshape(-1, 16).max(axis=1).astype(np.uint8)
    xs = O.f32_to_bf16_bits(x[2000:])
    for T in (600, 13):
        out.append((p, pc, T, O.encode(xs[:T], p, pc, 0, 0).stream))
    return out


def check_rans_golden():
    gd = golden("rans_examples.json")
    for case in gd["cases"]:
        sym = np.array(case["symbols"], np.uint8)
        states = case["states"] + [case["rest"]] * (64 - len(case["states"]))
        want = [v for pair in states for v in pair] + case["words"]
        (pay,) = LZ.rans_encode([sym], np.array(case["freq"]))
        assert pay.tolist() == want, (case["note"], pay.tolist())
        (back,) = LZ.rans_decode([pay], [len(sym)], np.array(case["freq"]))
        assert np.array_equal(back, sym)
    for case in gd["normalize"]:
        assert LZ.normalize(np.array(case["hist"])).tolist() == case["freq"], case


def check_rans_roundtrip_and_bound():
    """Random sources: the model sums to M with a slot for exactly the present
    symbols; decoding gives the chunk back; a chunk's payload is at most its
    static-model information plus the rANS slack (each symbol at most
    log2(17/16) bits above log2(M/f), since a state is at least 16 f) plus,
    per state, its 32-bit final value and one 16-bit word."""
    rng = np.random.default_rng(8)
    for A, n in ((2, 1), (4, 999), (16, 16384), (256, 40000), (256, 16385), (32, 2048)):
        sym = rng.choice(A, size=n, p=rng.dirichlet(np.full(A, 0.3))).astype(np.uint8)
        h = np.bincount(sym, minlength=A)
        f = LZ.normalize(h)
        assert f.sum() == LZ.M and np.array_equal(f > 0, h > 0)
        assert np.all(np.abs(f - h * LZ.M / n) <= np.count_nonzero(h) + 1)
        chunks = [sym[i:i + LZ.CHUNK] for i in range(0, n, LZ.CHUNK)]
        pays = LZ.rans_encode(chunks, f)
        for ch, pay, back in zip(chunks, pays, LZ.rans_decode(pays, [len(c) for c in chunks], f)):
            assert np.array_equal(ch, back)
            info = float(np.sum(np.log2(LZ.M / f[ch])))
            assert 16 * len(pay) <= info + len(ch) * np.log2(17 / 16) + 64 * 48, (A, n)


def check_lossless_fields():
    """The fields against the record parser: passthrough byte planes give the
    passthrough bytes, the shift and scale planes give the fp32 values, the
    code fields give each group's codes; merging them rebuilds the stream."""
    for p, sl, T, st in lossless_streams():
        fields = LZ.stream_fields(st, p, sl, T)
        esz = p.elem_bytes
        assert len(fields) == esz + 8 + sl.n_act
        s1, w1, tc = O.split_rows(T, p.sink, p.window)
        pt = np.stack([f for f, _ in fields[:esz]], axis=1).reshape(-1)
        assert pt.tobytes() == st[64:64 + (s1 + w1) * p.F * esz]
        codes, shift, scale = O.read_records(st, p, sl, T)
        sh = np.stack([f for f, _ in fields[esz:esz + 4]], axis=1).copy().view("<f4").reshape(tc, sl.n_act)
        sc = np.stack([f for f, _ in fields[esz + 4:esz + 8]], axis=1).copy().view("<f4").reshape(tc, sl.n_act)
        assert np.array_equal(sh.view(np.uint32), shift.view(np.uint32))
        assert np.array_equal(sc.view(np.uint32), scale.view(np.uint32))
        for a, g in enumerate(sl.active_groups):
            q, A = fields[esz + 8 + a]
            assert A == 1 << int(sl.widths[g])
            assert np.array_equal(q.reshape(tc, sl.G), codes[:, a * sl.G:(a + 1) * sl.G])
        assert LZ.merge_fields(st[:64], fields, p, sl, T) == st


def check_lossless_roundtrip():
    """Container round trip on every shape, within the stated bound."""
    for p, sl, T, st in lossless_streams():
        z = LZ.compress(st, p, sl, T)
        assert z[:4] == b"KVTZ" and len(z) <= LZ.container_bound(p, sl, T)
        assert LZ.decompress(z, p, sl, T) == st


_PC_ALLOCS = {}


def brute_force_pc(Dc, G, budgets, cap=None):
    """Every component width vector, ordered by (objective, bits of reading
    Q2c, largest component sum for the earliest group, lexicographically
    largest widths); the best one within each budget. Dc must hold exact
    binary fractions."""
    F, nb = Dc.shape
    n_g = F // G
    if (F, nb) not in _PC_ALLOCS:
        ws = np.array(list(itertools.product(range(nb), repeat=F)), np.int64)
        sums = ws.reshape(len(ws), n_g, G).sum(axis=2)
        cost = np.where(sums > 0, 64 + 8 * ((sums + 7) // 8), 0).sum(axis=1)
        _PC_ALLOCS[(F, nb)] = (ws, sums, cost)
    ws, sums, cost = _PC_ALLOCS[(F, nb)]
    if cap is not None:   # at most cap active groups
        keep = np.count_nonzero(sums, axis=1) <= cap
        ws, sums, cost = ws[keep], sums[keep], cost[keep]
    obj = np.sum(Dc[np.arange(F), ws], axis=1)
    keys = ([-ws[:, j] for j in range(F - 1, -1, -1)] + [-sums[:, g] for g in range(n_g - 1, -1, -1)]
            + [cost, obj])
    order = np.lexsort(keys)
    out = []
    for budget in budgets:
        i = order[np.argmax(cost[order] <= budget)]
        out.append(ws[i].astype(np.uint8))
    return out


def check_pc_pack_golden():
    gd = golden("pack_pc_examples.json")
    for case in gd["cases"]:
        q = np.array([case["codes"]], np.uint8)
        got = O.pack_codes_pc(q, case["widths"])
        assert got[0].tolist() == case["bytes"], (case["note"], got)
        back = O.unpack_codes_pc(got, case["widths"])
        want = [c if w else 0 for c, w in zip(case["codes"], case["widths"])]
        assert back[0].tolist() == want


def check_pc_quantizer_golden():
    gd = golden("quantizer_pc_examples.json")
    for case in gd["cases"]:
        c = np.array([case["c"]], np.float32)
        q, sh, sc = O.quantize_fp32_pc(c, case["widths"])
        assert q[0].tolist() == case["codes"], (case["note"], q)
        assert float(sh[0]) == case["shift"] and float(sc[0]) == case["scale"]
        ch = O.dequantize_pc(q, sh, sc, case["widths"])
        assert ch[0].tolist() == case["chat"], (case["note"], ch)


def check_pc_dp_bruteforce():
    """The per-component allocation of reading Q2c against brute force: one
    group of 8 components with widths 0..3, and two groups of 8 with widths
    0..1, also capped at one active group (reading Q3c); exact dyadic tables,
    ties included."""
    rng = np.random.default_rng(13)
    for trial in range(3):
        for n_g, nb in ((1, 4), (2, 2)):
            F = 8 * n_g
            e = np.sort(rng.uniform(0, 40, F))[::-1]
            Dc = np.array([[np.round(e[j] * 4.0 ** -b * 16) / 16 for b in range(nb)] for j in range(F)])
            if trial % 3 == 1:
                Dc[F // 2:] = Dc[:F // 2] if n_g == 2 else Dc[F // 2:]
            if trial % 3 == 2:
                Dc[-3:] = 0.0
            budgets = (0, 65, 72, 80, 90, 150, 170)
            for budget, bw in zip(budgets, brute_force_pc(Dc, 8, budgets)):
                w = O.dp_allocate_pc(Dc, 8, budget)
                assert np.array_equal(w, bw), (trial, n_g, budget, w, bw)
            if n_g == 2:   # reading Q3c: at most one active group
                for budget, bw in zip(budgets, brute_force_pc(Dc, 8, budgets, cap=1)):
                    w = O.dp_allocate_pc(Dc, 8, budget, max_active=1)
                    assert np.array_equal(w, bw), (trial, "cap 1", budget, w, bw)
                    assert np.array_equal(O._dp_allocate_pc_capped(Dc, 8, budget, 1), bw)


def check_pc_tables_and_reduction():
    """The per-component distortion table sums, over a group at one width,
    to the group table of reading Q2 (same grid, same quantizer); equal
    widths inside every group reproduce the group-width records byte for
    byte; per-component allocation is never worse than group widths; the
    quantizer keeps every coded component within half its step."""
    x, _ = family_b_small(seed=23, n=2400)
    p = small_params(F=64, G=16, bpv=3.0)
    sl = O.calibrate(x[:1600], p, 0, 0)
    rows = x[p.sink:1600 - p.window].astype(np.float64)
    C = (rows - sl.mu64) @ sl.V64
    Dc = O.distortion_table_pc(C, 16, 8)
    for g in range(4):
        for b in range(9):
            assert np.isclose(Dc[g * 16:(g + 1) * 16, b].sum(), sl.D[g, b], rtol=1e-12, atol=1e-300)
    eq = O.Slot(0, 0, 64, 16, sl.widths, sl.mu32, sl.lam, sl.V32,
                cwidths=np.repeat(sl.widths, 16).astype(np.uint8))
    assert eq.record_bytes == sl.record_bytes
    xe = x[1600:].astype(np.float32)
    a_ = O.encode(xe, p, sl, 0, 0).stream
    b_ = O.encode(xe, p, eq, 0, 0).stream
    assert a_[O.HEADER_BYTES:] == b_[O.HEADER_BYTES:]
    cw = O.dp_allocate_pc(Dc, 16, p.budget_bits)
    obj_pc = sum(Dc[j, b] for j, b in enumerate(cw))
    obj_g = sum(sl.D[g, b] for g, b in enumerate(sl.widths))
    assert obj_pc <= obj_g * (1 + 1e-12)
    pc = O.calibrate_set([(0, 0, x[:1600])], p, component_widths=True)[(0, 0)]
    assert np.array_equal(pc.cwidths, cw)
    er = O.encode(xe, p, pc, 0, 0)
    for a, g in enumerate(pc.active_groups):
        bs = pc.group_cwidths(g)
        cg = er.coeffs[:, a * 16:(a + 1) * 16].astype(np.float64)
        ch = O.dequantize_pc(er.codes[:, a * 16:(a + 1) * 16], er.shift[:, a], er.scale[:, a], bs)
        for j, b in enumerate(bs):
            if b:
                step = er.scale[:, a].astype(np.float64) / (2 ** int(b) - 1)
                assert np.all(np.abs(cg[:, j] - ch[:, j]) <= step / 2 * (1 + 1e-5) + 1e-6 * np.abs(cg[:, j]))
            else:
                assert np.all(ch[:, j] == 0)
    art = O.parse_artifact(O.Artifact(p, {(0, 0): pc}).serialize()).slots[(0, 0)]
    assert np.array_equal(art.cwidths, pc.cwidths) and art.record_bytes == pc.record_bytes


def check_projection_exact():
    """c = fp32 of the exact sum of (x - mu32) times bf16 V' (section 2B)."""
    rng = np.random.default_rng(6)
    F, r = 64, 32
    V32 = np.linalg.qr(rng.standard_normal((F, F)))[0][:, :r].astype(np.float32)
    mu = rng.standard_normal(F).astype(np.float32)
    sl = injected_slot(V32, [1, 1, 0, 0], mu, 16)
    x = (rng.standard_normal((5, F)) * 3 + mu).astype(np.float32)
    c = O.project(x, sl)
    import torch
    Vb = torch.from_numpy(V32).to(torch.bfloat16).double().numpy()
    for t in range(5):
        for j in range(r):
            exact = sum((fractions.Fraction(float(x[t, f])) - fractions.Fraction(float(mu[f]))) *
                        fractions.Fraction(float(Vb[f, j])) for f in range(F))
            assert c[t, j] == np.float32(float(exact)), (t, j)


def check_exact_roundtrip_identity():
    """mu = 0, V = I, all groups at 8 bits, values on each group's 8-bit grid:
    decode returns the input bit for bit."""
    rng = np.random.default_rng(8)
    F, G, T = 64, 16, 40
    p = small_params(F=F, G=G, bpv=12.0)
    sl = injected_slot(np.eye(F), [8, 8, 8, 8], np.zeros(F), G)
    x = np.zeros((T, F), np.float32)
    for g in range(F // G):
        e = rng.integers(-6, 3, T).astype(np.float64)
        m = rng.integers(-255, 1, T)               # |m + q| <= 255 is exact in bf16
        q = rng.integers(0, 256, (T, G))
        q[:, 0], q[:, 1] = 0, 255
        x[:, g * G:(g + 1) * G] = (m[:, None] + q) * 2.0 ** e[:, None]
    assert np.array_equal(O.bf16_rne(x), x)
    er = O.encode(x, p, sl, 0, 0)
    full, out = O.decode(er.stream, p, sl, 0, 0, T)
    assert np.array_equal(out.view(np.uint32), x.view(np.uint32)), "identity round trip not exact"


def check_hadamard_roundtrip_bound():
    """Exactly orthonormal bf16 basis (Hadamard / 8): ||x_hat - mu - x'|| <=
    sqrt(sum (step/2)^2), by Parseval and the half-step bound."""
    rng = np.random.default_rng(9)
    F, G, T = 64, 16, 300
    H = hadamard(F) / 8.0
    assert np.allclose(H.T @ H, np.eye(F))
    mu = rng.standard_normal(F).astype(np.float32)
    for widths in ([8, 8, 8, 8], [6, 4, 2, 1], [3, 0, 5, 0]):
        p = small_params(F=F, G=G, bpv=12.0, s=2, w=3)
        cols = [j for g in range(4) if widths[g] for j in range(g * G, (g + 1) * G)]
        sl = injected_slot(H[:, cols], widths, mu, G)
        x = (rng.standard_normal((T, F)) * 2 + mu).astype(np.float32)
        er = O.encode(x, p, sl, 0, 0)
        full, _ = O.decode(er.stream, p, sl, 0, 0, T)
        xs = x[2:T - 3]
        xprime = xs.astype(np.float64) - mu.astype(np.float64)
        err = full[2:T - 3] - mu.astype(np.float64) - xprime
        bound2 = np.zeros(T - 5)
        act = [g for g in range(4) if widths[g]]
        for a, g in enumerate(act):
            step = er.scale[:, a].astype(np.float64) / (2 ** widths[g] - 1)
            bound2 += G * (step / 2) ** 2
        for g in range(4):
            if not widths[g]:
                bound2 += np.sum((xprime @ H[:, g * G:(g + 1) * G]) ** 2, axis=1)
        assert np.all(np.sum(err ** 2, axis=1) <= bound2 * (1 + 1e-3) + 1e-12), widths


def check_zero_bit_decodes_to_mean():
    rng = np.random.default_rng(10)
    F, T = 64, 50
    for dtype in (O.DTYPE_F32, O.DTYPE_BF16):
        p = small_params(F=F, dtype=dtype, s=3, w=5)
        mu = rng.standard_normal(F).astype(np.float32)
        sl = injected_slot(np.zeros((F, 0)), [0, 0, 0, 0], mu, 16)
        x = rng.standard_normal((T, F)).astype(np.float32)
        store = O.f32_to_bf16_bits(x) if dtype == O.DTYPE_BF16 else x
        er = O.encode(store, p, sl, 0, 0)
        assert sl.record_bytes == 0
        for od in (O.DTYPE_F32, O.DTYPE_BF16):
            full, out = O.decode(er.stream, p, sl, 0, 0, T, od)
            want = O.f32_to_bf16_bits(mu) if od == O.DTYPE_BF16 else mu
            assert np.array_equal(out[3:T - 5], np.broadcast_to(want, (T - 8, F)))
            if od == dtype:
                assert np.array_equal(out[:3], store[:3]) and np.array_equal(out[T - 5:], store[T - 5:])


def check_sink_window_layout():
    rng = np.random.default_rng(11)
    F = 64
    mu = np.zeros(F, np.float32)
    sl = injected_slot(np.eye(F)[:, :16], [4, 0, 0, 0], mu, 16)
    for T, s, w in ((100, 4, 8), (12, 4, 8), (10, 4, 8), (3, 4, 8), (0, 4, 8), (30, 0, 0)):
        p = small_params(F=F, s=s, w=w, dtype=O.DTYPE_BF16)
        x = O.f32_to_bf16_bits(rng.standard_normal((T, F)).astype(np.float32))
        er = O.encode(x, p, sl, 0, 0)
        h = O.parse_header(er.stream)
        s1 = min(s, T)
        w1 = min(w, T - s1)
        assert (h.s, h.w, h.tc) == (s1, w1, T - s1 - w1)
        pt = np.frombuffer(er.stream, np.uint16, (s1 + w1) * F, 64).reshape(-1, F)
        assert np.array_equal(pt[:s1], x[:s1]) and np.array_equal(pt[s1:], x[T - w1:])
        assert len(er.stream) == 64 + (s1 + w1) * F * 2 + (T - s1 - w1) * sl.record_bytes
        full, out = O.decode(er.stream, p, sl, 0, 0, T, O.DTYPE_BF16)
        assert np.array_equal(out[:s1], x[:s1]) and np.array_equal(out[T - w1:], x[T - w1:])


def check_header_golden():
    gd = golden("header_example.json")
    f = gd["fields"]

    class FakeSlot:
        G = f["G"]
        n_act = len(f["widths_active"])
        record_bytes = 8 * n_act + f["G"] * sum(f["widths_active"]) // 8
        slot_id = int(f["slot_id"], 16)

    p = O.Params(8, 8, 128, f["sink"], f["window"], f["G"], 8, 1.0, f["dtype"])
    h = O.make_header(p, FakeSlot, f["layer"], f["kind"], f["T"])
    assert h.hex() == gd["hex"].replace(" ", ""), h.hex()
    assert FakeSlot.record_bytes == gd["derived"]["record_bytes"]


def check_header_validation():
    rng = np.random.default_rng(12)
    F, T = 64, 40
    p = small_params(F=F)
    sl = injected_slot(np.eye(F)[:, :16], [4, 0, 0, 0], np.zeros(F, np.float32), 16)
    er = O.encode(rng.standard_normal((T, F)).astype(np.float32), p, sl, 2, 1)
    O.decode(er.stream, p, sl, 2, 1, T)
    bad = []
    for off in (0, 4, 6, 7, 8, 12, 16, 20, 24, 28, 32, 34, 36, 40, 47):
        s = bytearray(er.stream)
        s[off] ^= 0x5A
        bad.append(bytes(s))
    for s in bad:
        try:
            O.decode(s, p, sl, 2, 1, T)
        except O.OracleError:
            continue
        raise AssertionError("corrupt header accepted")
    for args in ((3, 1, T), (2, 0, T), (2, 1, T + 1)):
        try:
            O.decode(er.stream, p, sl, *args)
        except O.OracleError:
            continue
        raise AssertionError("mismatched job accepted")
    try:
        O.decode(er.stream[:-1], p, sl, 2, 1, T)
    except O.OracleError:
        pass
    else:
        raise AssertionError("truncated stream accepted")


def check_artifact_roundtrip():
    x, _ = family_b_small(seed=13, n=1024)
    p = O.Params(1, 2, 32, 4, 8, 16, 8, 2.0, O.DTYPE_F32)
    sl = O.calibrate(x, p, 0, 1)
    art = O.Artifact(p, {(0, 1): sl})
    buf = art.serialize()
    back = O.parse_artifact(buf)
    s2 = back.slots[(0, 1)]
    assert np.array_equal(s2.widths, sl.widths) and np.array_equal(s2.V32, sl.V32)
    assert np.array_equal(s2.mu32, sl.mu32) and np.array_equal(s2.lam, sl.lam)
    assert s2.slot_id == sl.slot_id
    raw = bytearray(buf)
    raw[-20] ^= 1
    try:
        O.parse_artifact(bytes(raw))
    except O.OracleError:
        pass
    else:
        raise AssertionError("corrupt artifact accepted")
    # layout: slot header and widths at the documented offsets
    assert buf[48:52] == b"KVTS"
    assert struct.unpack_from("<7i", buf, 52)[:6] == (0, 1, 64, 16, sl.n_act, sl.r_eff)


def check_decode_exact_sum():
    """x_hat = mu32 + sum_j c_hat_j V'_j, checked element-wise in exact rationals."""
    rng = np.random.default_rng(14)
    F, T = 64, 30
    V32 = np.linalg.qr(rng.standard_normal((F, F)))[0][:, :32].astype(np.float32)
    mu = rng.standard_normal(F).astype(np.float32)
    p = small_params(F=F, s=1, w=1)
    sl = injected_slot(V32, [3, 0, 6, 0], mu, 16)
    x = (rng.standard_normal((T, F)) + mu).astype(np.float32)
    er = O.encode(x, p, sl, 0, 0)
    full, _ = O.decode(er.stream, p, sl, 0, 0, T)
    import torch
    Vb = torch.from_numpy(sl.V32).to(torch.bfloat16).double().numpy()
    Fr = fractions.Fraction
    for t in (0, 7, 27):
        for f in (0, 13, 63):
            acc = Fr(float(mu[f]))
            for a, b in ((0, 3), (1, 6)):
                step = np.float32(er.scale[t, a]) / np.float32(2 ** b - 1)
                for j in range(16):
                    chat = Fr(float(er.shift[t, a])) + int(er.codes[t, 16 * a + j]) * Fr(float(step))
                    acc += chat * Fr(float(Vb[f, 16 * a + j]))
            assert abs(float(acc) - full[t + 1, f]) <= 1e-12 * max(1.0, abs(float(acc)))


def check_deflate_ratio():
    """Z1: DEFLATE is lossless (inflate gives the stream back), the ratios are
    raw bytes over stream bytes and over deflated bytes, and the level is 6:
    a zlib stream (RFC 1950) starts with CMF = 0x78 (deflate, 32 KiB window)
    and an FLG byte whose top two bits are the level class, 2 ("default")
    for level 6, which with the check bits gives 0x9C."""
    import zlib
    rng = np.random.default_rng(12)
    stream = bytes(2000) + rng.integers(0, 4, 3000, dtype=np.uint8).tobytes() + b"KVTC" * 250
    assert len(stream) == 6000
    r_stream, r_defl, z = O.deflate_ratio(stream, 96000)
    assert zlib.decompress(z) == stream
    assert r_stream == 16.0
    assert r_defl == 96000 / len(z) and len(z) < 3000
    assert z[0] == 0x78 and z[1] == 0x9C and (z[0] * 256 + z[1]) % 31 == 0


def check_shapes_vs_page():
    w = synth.workload("llama31_8b")
    per_1k = w.n_layers * len(w.kinds) * w.features * 2 * 1024
    assert per_1k == 128 * 2 ** 20, "Llama 3.1 8B KV at 1K tokens must be 128 MiB"


def check_generators():
    w = synth.workload("tiny")
    a = synth.gen_kv(w, 0, 0, 1, 300)
    b = synth.gen_kv(w, 0, 0, 1, 300)
    c = synth.gen_kv(w, 0, 0, 2, 300)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    x = synth.gen_kv(w, 0, 0, 1, 4000).astype(np.float64)
    ev = np.linalg.eigvalsh(np.cov(x.T))[::-1]
    assert ev[15] > 50 * ev[16], "family A must have rank 16 above the noise"
    wb = synth.workload("llama31_8b")
    y = synth.gen_kv(wb, 0, 0, 1, 64)
    assert np.array_equal(O.bf16_rne(y), y)


ALL = [v for k, v in sorted(globals().items()) if k.startswith("check_")]
