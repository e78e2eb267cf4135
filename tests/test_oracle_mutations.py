"""Plant plausible mistakes in the CPU oracle and show that the pins catch them.

Every mutation here is applied to the oracle module only, on the CPU, for the
duration of one test.  Each must make at least one of the listed pin checks
fail; that is what makes the pins a real check of the oracle rather than a
restatement of it.
"""
import numpy as np
import pytest

import oracle.kvtc_lossless as LZ
import oracle.kvtc_oracle as O
import pins

_orig = {name: getattr(O, name) for name in dir(O) if callable(getattr(O, name))}
_orig_lz = {name: getattr(LZ, name) for name in dir(LZ) if callable(getattr(LZ, name))}


def _project_no_centering(x_vals, slot):
    xc = x_vals.astype(np.float64)
    return (xc @ slot.basis_bf16().astype(np.float64)).astype(np.float32)


def _project_fp32_basis(x_vals, slot):
    xc = x_vals.astype(np.float64) - slot.mu32.astype(np.float64)
    return (xc @ slot.V32.astype(np.float64)).astype(np.float32)


def _project_bf16_centred(x_vals, slot):
    xc = O.bf16_rne((x_vals.astype(np.float32) - slot.mu32).astype(np.float32))
    return (xc.astype(np.float64) @ slot.basis_bf16().astype(np.float64)).astype(np.float32)


def _dequant_wrong_levels(q, shift, scale, b):
    step = (np.asarray(scale, np.float32) / np.float32(2 ** b)).astype(np.float32)
    return shift.astype(np.float64)[:, None] + q * step.astype(np.float64)[:, None]


def _dequant_wrong_sign(q, shift, scale, b):
    return -_orig["dequantize"](q, -shift, scale, b) + 0.0 * q


def _pack_msb_first(q, b):
    T, G = q.shape
    bits = ((q.astype(np.uint16)[:, :, None] >> np.arange(b - 1, -1, -1, dtype=np.uint16)) & 1)
    return np.packbits(bits.astype(np.uint8).reshape(T, G * b), axis=1, bitorder="little")


def _split_swapped(T, s, w):
    return _orig["split_rows"](T, w, s)


def _pca_unsorted(xc):
    V, lam = _orig["pca_basis"](xc)
    return V[:, ::-1].copy(), lam[::-1].copy()


def _pca_no_sign(xc):
    n, F = xc.shape
    _, s, vt = np.linalg.svd(xc, full_matrices=n < F)
    V = -vt.T
    return V, s ** 2 / n


def _dp_small_lex(D, G, budget):
    """Ties resolved toward the smallest widths instead of the largest."""
    n_g, nb = D.shape
    f = np.full((n_g + 1, budget + 1), np.inf)
    f[n_g, 0] = 0.0
    for g in range(n_g - 1, -1, -1):
        for u in range(budget + 1):
            for b in range(nb):
                c = O.group_cost(b, G)
                if c <= u:
                    f[g, u] = min(f[g, u], D[g, b] + f[g + 1, u - c])
    u = int(np.argmin(f[0]))
    w = np.zeros(n_g, np.uint8)
    for g in range(n_g):
        for b in range(nb):
            c = O.group_cost(b, G)
            if c <= u and D[g, b] + f[g + 1, u - c] == f[g, u]:
                w[g] = b
                u -= c
                break
    return w


def _dp_no_scale_cost(D, G, budget):
    old = O.group_cost
    try:
        O.group_cost = lambda b, G: G * b
        return _orig["dp_allocate"](D, G, budget)
    finally:
        O.group_cost = old


def _quant_floor(c, b):
    c = np.asarray(c, np.float32)
    k = np.float32(2 ** b - 1)
    shift = c.min(axis=1)
    scale = (c.max(axis=1) - shift).astype(np.float32)
    nz = scale > 0
    inv = np.zeros_like(scale)
    inv[nz] = k / scale[nz]
    u = ((c - shift[:, None]).astype(np.float32) * inv[:, None]).astype(np.float32)
    q = np.clip(np.floor(u), 0, k)
    q[~nz] = 0
    return q.astype(np.uint8), shift, scale


def _reconstruct_no_mean(codes, shift, scale, slot):
    return _orig["reconstruct"](codes, shift, scale, slot) - slot.mu32.astype(np.float64)


def _distortion_dropped_term(C, G, max_bits):
    D = _orig["distortion_table"](C, G, max_bits)
    D[:, 0] = 0.0
    return D


def _calibrate_all_rows(x_cal, params, layer, kind):
    p2 = O.Params(**{**params.__dict__, "sink": 0, "window": 0})
    return _orig["calibrate"](x_cal, p2, layer, kind)


def _bf16_truncate(x):
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((b >> 16) << 16).view(np.float32).reshape(np.shape(x))


def _header_swapped(params, slot, layer, kind, T):
    p2 = O.Params(**{**params.__dict__, "sink": params.window, "window": params.sink})
    return _orig["make_header"](p2, slot, layer, kind, T)


def _quant_no_clamp(c, b):
    q, shift, scale = _orig["quantize_fp32"](c, b)
    return np.where(q == 2 ** b - 1, 0, q).astype(np.uint8), shift, scale


def _deflate_level9(stream, raw_bytes):
    import zlib
    z = zlib.compress(bytes(stream), 9)
    return raw_bytes / len(stream), raw_bytes / len(z), z


def _deflate_ratios_swapped(stream, raw_bytes):
    a, b, z = _orig["deflate_ratio"](stream, raw_bytes)
    return b, a, z


def _global_latest_first(Ds, G, budget, max_active):
    """Ties between tensors resolved toward the last tensor."""
    return _orig["dp_allocate_global"](Ds[::-1], G, budget, max_active)[::-1]


def _global_cap_ignored(Ds, G, budget, max_active):
    return _orig["dp_allocate_global"](Ds, G, budget, max(D.shape[0] for D in Ds))


def _global_per_tensor(Ds, G, budget, max_active):
    return [O.dp_allocate(D, G, budget) for D in Ds]


def _shared_pooled_mean(rows_list):
    x = np.vstack(rows_list)
    return O.pca_basis(x - x.mean(axis=0))


def _shared_first_only(rows_list):
    return O.pca_basis(rows_list[0] - rows_list[0].mean(axis=0))


def _calibrate_set_kinds_pooled(inputs, params, shared_basis=False, global_budget=False,
                                max_active=None):
    """K and V pooled into one shared basis."""
    out = _orig["calibrate_set"]([(2 * l + k, 0, x) for l, k, x in inputs], params,
                                 shared_basis, global_budget, max_active)
    res = {}
    for (lk, _), sl in out.items():
        sl.layer, sl.kind = lk // 2, lk % 2
        res[(lk // 2, lk % 2)] = sl
    return res


def _normalize_remainder_to_first(hist):
    f = _orig_lz["normalize"](hist)
    h = np.asarray(hist)
    if h.sum():
        r = int(np.argmax(h))
        first = int(np.argmax(h > 0))
        extra = f[r] - (1 + (h[r] * (LZ.M - np.count_nonzero(h))) // h.sum())
        f[r] -= extra
        f[first] += extra
    return f


def _normalize_no_floor_one(hist):
    h = np.asarray(hist, np.int64)
    f = np.zeros(h.size, np.int64)
    if h.sum():
        f = (h * LZ.M) // h.sum()
        f[int(np.argmax(h))] += LZ.M - int(f.sum())
    return f


def _interleaved_encode(chunks, f, late=False, descending=False):
    """The chunk coder with one planted change: renormalise when x > f * 2^20
    instead of >= (late), or order a step's words by descending lane."""
    f = np.asarray(f, np.int64)
    c = np.concatenate([[0], np.cumsum(f)[:-1]])
    out = []
    for ch in chunks:
        n = len(ch)
        x = [LZ.RANS_L] * LZ.LANES
        groups = []
        for t in range((n + LZ.LANES - 1) // LZ.LANES - 1, -1, -1):
            words = []
            for l in range(LZ.LANES):
                i = t * LZ.LANES + l
                if i >= n:
                    continue
                fs, cs = int(f[ch[i]]), int(c[ch[i]])
                if (x[l] > (fs << 20)) if late else (x[l] >= (fs << 20)):
                    words.append(x[l] & 0xFFFF)
                    x[l] >>= 16
                x[l] = (x[l] // fs) * LZ.M + x[l] % fs + cs
            groups.append(words[::-1] if descending else words)
        states = [v for xl in x for v in (xl & 0xFFFF, xl >> 16)]
        out.append(np.array(states + [w for g in groups[::-1] for w in g], np.uint64).astype(np.uint16))
    return out


def _rans_emit_late(chunks, f):
    return _interleaved_encode(chunks, f, late=True)


def _rans_words_descending(chunks, f):
    return _interleaved_encode(chunks, f, descending=True)


def _fields_planes_big_endian(stream, params, slot, T):
    fs = _orig_lz["stream_fields"](stream, params, slot, T)
    esz = params.elem_bytes
    return fs[:esz][::-1] + fs[esz:esz + 4][::-1] + fs[esz + 4:esz + 8][::-1] + fs[esz + 8:]


def _fields_codes_component_major(stream, params, slot, T):
    fs = _orig_lz["stream_fields"](stream, params, slot, T)
    esz = params.elem_bytes
    out = fs[:esz + 8]
    for q, A in fs[esz + 8:]:
        out.append((q.reshape(-1, slot.G).T.reshape(-1).copy(), A))
    return out


def _fields_pc_alphabet_first_width(stream, params, slot, T):
    fs = _orig_lz["stream_fields"](stream, params, slot, T)
    if getattr(slot, "cwidths", None) is None:
        return fs
    esz = params.elem_bytes
    out = fs[:esz + 8]
    for (q, _), g in zip(fs[esz + 8:], slot.active_groups):
        out.append((q, 1 << int(slot.group_cwidths(g)[0])))
    return out


def _pack_pc_msb_first(q, bs):
    rev = q.copy()
    for j, b in enumerate(bs):
        if b:
            v = q[:, j].astype(np.uint16)
            rev[:, j] = sum(((v >> i) & 1) << (int(b) - 1 - i) for i in range(int(b))).astype(np.uint8)
    return _orig["pack_codes_pc"](rev, bs)


def _dequant_pc_group_width(q, shift, scale, bs):
    m = int(np.max(bs))
    return _orig["dequantize_pc"](q, shift, scale, [m if b else 0 for b in bs])


def _quant_pc_active_range(c, bs):
    """Shift and scale over the coded components only."""
    c = np.asarray(c, np.float32)
    act = np.asarray(bs) > 0
    q, _, _ = _orig["quantize_fp32_pc"](c[:, act], np.asarray(bs)[act])
    full = np.zeros(c.shape, np.uint8)
    full[:, act] = q
    shift = c[:, act].min(axis=1)
    return full, shift, (c[:, act].max(axis=1) - shift).astype(np.float32)


def _group_cost_pc_unpadded(s_):
    return 0 if s_ == 0 else 64 + s_


def _dp_pc_cap_ignored(Dc, G, budget, max_active=None):
    return _orig["dp_allocate_pc"](Dc, G, budget)


def _dp_pc_capped_counts_all_groups(Dc, G, budget, max_active):
    """The cap charged for every group, active or not."""
    return _orig["_dp_allocate_pc_capped"](Dc, G, budget, max(0, max_active - Dc.shape[0] // G + 1))


PC_MUTATIONS = {
    "pc_cap_ignored": ("dp_allocate_pc", _dp_pc_cap_ignored),
    "pc_cap_counts_all_groups": ("_dp_allocate_pc_capped", _dp_pc_capped_counts_all_groups),
    "pc_pack_msb_first": ("pack_codes_pc", _pack_pc_msb_first),
    "pc_dequant_group_width": ("dequantize_pc", _dequant_pc_group_width),
    "pc_range_over_coded_only": ("quantize_fp32_pc", _quant_pc_active_range),
    "pc_cost_without_padding": ("group_cost_pc", _group_cost_pc_unpadded),
}


LZ_MUTATIONS = {
    "lz_normalize_remainder_to_first": ("normalize", _normalize_remainder_to_first),
    "lz_normalize_drops_rare": ("normalize", _normalize_no_floor_one),
    "lz_rans_emit_late": ("rans_encode", _rans_emit_late),
    "lz_rans_word_order": ("rans_encode", _rans_words_descending),
    "lz_planes_big_endian": ("stream_fields", _fields_planes_big_endian),
    "lz_codes_component_major": ("stream_fields", _fields_codes_component_major),
    "lz_pc_alphabet_first_width": ("stream_fields", _fields_pc_alphabet_first_width),
}


MUTATIONS = {
    "global_ties_to_last_tensor": ("dp_allocate_global", _global_latest_first),
    "global_cap_ignored": ("dp_allocate_global", _global_cap_ignored),
    "global_budget_per_tensor": ("dp_allocate_global", _global_per_tensor),
    "shared_basis_pooled_mean": ("shared_pca", _shared_pooled_mean),
    "shared_basis_first_tensor": ("shared_pca", _shared_first_only),
    "shared_basis_kinds_pooled": ("calibrate_set", _calibrate_set_kinds_pooled),
    "deflate_level9": ("deflate_ratio", _deflate_level9),
    "deflate_ratios_swapped": ("deflate_ratio", _deflate_ratios_swapped),
    "no_centering": ("project", _project_no_centering),
    "fp32_basis_in_projection": ("project", _project_fp32_basis),
    "bf16_centred_operand": ("project", _project_bf16_centred),
    "dequant_wrong_levels": ("dequantize", _dequant_wrong_levels),
    "dequant_wrong_sign": ("dequantize", _dequant_wrong_sign),
    "pack_msb_first": ("pack_codes", _pack_msb_first),
    "sink_window_swapped": ("split_rows", _split_swapped),
    "pca_unsorted": ("pca_basis", _pca_unsorted),
    "pca_no_sign_rule": ("pca_basis", _pca_no_sign),
    "dp_no_scale_cost": ("dp_allocate", _dp_no_scale_cost),
    "dp_ties_smallest": ("dp_allocate", _dp_small_lex),
    "quant_floor": ("quantize_fp32", _quant_floor),
    "quant_top_code_lost": ("quantize_fp32", _quant_no_clamp),
    "reconstruct_no_mean": ("reconstruct", _reconstruct_no_mean),
    "distortion_dropped_term": ("distortion_table", _distortion_dropped_term),
    "calibrate_all_rows": ("calibrate", _calibrate_all_rows),
    "bf16_truncate": ("bf16_rne", _bf16_truncate),
    "header_fields_swapped": ("make_header", _header_swapped),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS) + sorted(PC_MUTATIONS) + sorted(LZ_MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    if name in LZ_MUTATIONS:
        attr, fake = LZ_MUTATIONS[name]
        monkeypatch.setattr(LZ, attr, fake)
    else:
        attr, fake = {**MUTATIONS, **PC_MUTATIONS}[name]
        monkeypatch.setattr(O, attr, fake)
    failed = []
    for check in pins.ALL:
        try:
            check()
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            failed.append(check.__name__)
    assert failed, f"mutation {name} was not caught by any pin"
