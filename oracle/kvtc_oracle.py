"""Plain, slow, CPU oracle of KV-cache transform coding (KVTC).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke entry point and by
the CPU-baseline leg of the benchmark.  The HIP library never imports, links or
calls anything here, and this module shares no code with it; the two meet only
through the byte formats written out below.

Source: the page "KV Cache Transform Coding for Compact Storage in LLM
Inference" (gist.science, paper 2511.01815), section 2 (methodology):
  2A calibration  - PCA of calibration KV through an SVD gives an orthonormal
                    basis V, computed once and shared across heads; the oldest s
                    (sink) and newest w (window) tokens are not compressed; a
                    dynamic program assigns each principal component a bit width
                    under a bit budget (high-variance components get more bits,
                    low-variance ones get 0 bits and are dropped); a group of
                    components shares a scale and a shift (microscaling).
  2B compression  - subtract the mean, multiply by V, quantize with the DP
                    widths, pack the integers, then DEFLATE.
  2C decompression- the exact reverse: inflate, dequantize, multiply by V^T,
                    add the mean.

The pages give no formula, bit layout, rounding rule or tie-break.  Each such
choice below is marked READING and is the plainest one the text supports:

  R1  calibration rows are [s, n - w), the rows that would be compressed.
  R2  components sorted by descending singular value (stable by index); each
      basis column's largest-magnitude entry made positive (lowest index wins
      a tie).
  P1  one basis per (layer, K|V) over the concatenated kv_heads*head_dim
      features (shared across heads).
  Q1  uniform affine grid per group: "scale and shift" define it; the
      quantization is non-uniform across groups through their widths.
  Q2  one width per microscale group of G consecutive components.
  Q3  widths b in {0..8}.
  Q4  shift = group minimum and scale = group range, per (token, group),
      stored as two fp32 values (64 bits) counted in the budget.
  Q5  the DP's distortion is the empirical squared error of that quantizer
      (in fp64) on the calibration coefficients.
  Q6  budget B = floor(bits_per_value * F) bits per compressed token, shift and
      scale included, sink and window excluded.
  Q7  DP ties: fewest total bits, then the lexicographically largest widths.
  N1  projection c = fp32 of sum_f (x_f - mu32_f) V'_fj, the centred values
      and the sum taken exactly (fp64 here: x - mu32 is exact in fp64);
      operational basis V' = bf16_rne(fp32(V)) restricted to active groups.
  N2  round half to even; clamp to [0, 2^b - 1]; a zero range gives code 0;
      IEEE fp32 division; no fused multiply-add in the quantizer.
  Z0  a dropped (0-bit) component decodes to 0, so it adds nothing to the mean.
  Z1  DEFLATE is zlib level 6 over the whole stream, for the ratio only.

Calibration of a set of tensors at once (calibrate_set), for the page's
claims that one basis serves several layers and heads (section 3, second
contribution) and that the DP places bits where they lower the error most
(section 2A):
  P1s shared basis: the tensors of one kind (K or V) in the set share one
      basis V, the PCA of their pooled rows, each tensor's rows centred on its
      own mean first; each tensor keeps its own mean, distortion table and
      widths.
  Q6g global budget: the widths of every tensor in the set are chosen
      together, minimising the sum of their distortions subject to the sum of
      their bits per token being at most (number of tensors) * B; every tensor
      compresses the same tokens, so this is the same total size as B each.
      A tensor may hold at most max_active active groups (the library's
      records index at most 256 components).
  Q7g ties of the global allocation: fewest total bits, then the most bits to
      the tensor earliest in (layer, kind) order, then Q7 inside each tensor.

Per-component widths (the page's section 2A gives each principal component
its own width; READING Q2c, an alternative to Q2 chosen at calibration):
  Q2c every component j of a group has its own width b_j in 0..max_bits; the
      group's (shift, scale) is the min and range of all G of its components
      per token, as in Q4; component j is coded on 2^b_j - 1 levels of that
      range (q = clamp(rint(fp32(c - shift) * fp32(k_j / scale)), 0, k_j)) and
      decodes to shift + q * fp32(scale / k_j); b_j = 0 drops it (it decodes
      to 0).  A group is active if any b_j > 0.  Its codes are packed in
      component order, code j at bit sum_{i<j} b_i of the group's chunk, LSB
      first; the chunk is ceil(sum_j b_j / 8) bytes (zero padded).  Cost of
      an active group: 64 + 8 * ceil(sum_j b_j / 8) bits.  Distortion D_j(b):
      the empirical error of that quantizer on component j with its group's
      grid.  DP: per group, E_g(s) = least sum_j D_j(b_j) with sum_j b_j = s;
      across groups, least sum_g E_g(s_g) within the budget.  Ties: fewest
      bits, then the largest s for the earliest group, then the
      lexicographically largest widths inside a group.  Slot format: the
      seventh header int is 1 and the widths array holds F component widths.
  Q3c with a cap of max_active active groups (the library's 256 components),
      used only when the plain allocation breaks it: the across-group DP also
      counts the active groups, f[g][u][r] = least distortion of groups g.. at
      exactly u bits with at most r active; the same tie order.

Byte formats (all little-endian):

  artifact  = "KVTA" u32 version, i32 n_layers, kv_heads, head_dim, sink,
              window, group, max_bits, f32 bits_per_value, i32 dtype,
              i32 n_slots, then n_slots slot blocks.
  slot      = "KVTS", i32 layer, kind, F, G, n_act, r_eff, 0,
              u8 widths[F/G] zero-padded to a multiple of 8,
              f32 mu32[F], f64 lambda[F], f32 V32[F][r_eff] (active columns in
              component order), u64 slot_id = FNV-1a-64 of the slot's preceding
              bytes.
  stream    = 64-byte header, then the raw passthrough rows [0, s') and
              [T - w', T), then T_c records.
  header    = "KVTC", u16 version, u8 dtype, u8 kind, u32 layer, T, F, s', w',
              T_c, u16 G, u16 n_act, u32 record_bytes, u64 slot_id, zeros.
  record    = n_act pairs (f32 shift, f32 scale), then for each active group
              its G codes, code j at bits [j*b, j*b + b) of the group's chunk,
              least significant bit first (stream bit n = bit n%8 of byte n/8).
"""
from __future__ import annotations

import dataclasses
import struct
import zlib

import numpy as np

DTYPE_F32, DTYPE_BF16 = 0, 1
KIND_K, KIND_V = 0, 1
STREAM_MAGIC = b"KVTC"
ART_MAGIC = b"KVTA"
SLOT_MAGIC = b"KVTS"
FORMAT_VERSION = 1
HEADER_BYTES = 64
SCALE_BITS = 64          # fp32 shift + fp32 scale per active group (Q4)


class OracleError(ValueError):
    pass


# ---------------------------------------------------------------- numerics ---

def bf16_rne(x) -> np.ndarray:
    """Round fp32 values to the nearest bfloat16 (ties to even); fp32 result."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    keep = b >> 16
    rem = b & 0xFFFF
    up = (rem > 0x8000) | ((rem == 0x8000) & ((keep & 1) == 1))
    out = ((keep + up.astype(np.uint64)) << 16).astype(np.uint32)
    return out.view(np.float32).reshape(np.shape(x))


def bf16_to_f32(bits) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(x) -> np.ndarray:
    return (bf16_rne(x).view(np.uint32) >> 16).astype(np.uint16)


def fnv1a64(data: bytes) -> int:
    """FNV-1a, 64-bit (offset basis 0xcbf29ce484222325, prime 2^40 + 2^8 + 0xb3)."""
    h = 0xCBF29CE484222325
    for byte in data:
        h ^= byte
        h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h


# ------------------------------------------------------------------ params ---

@dataclasses.dataclass
class Params:
    n_layers: int
    kv_heads: int
    head_dim: int
    sink: int
    window: int
    group: int
    max_bits: int
    bits_per_value: float
    dtype: int

    @property
    def F(self) -> int:
        return self.kv_heads * self.head_dim

    @property
    def n_groups(self) -> int:
        return self.F // self.group

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == DTYPE_F32 else 2

    @property
    def budget_bits(self) -> int:
        # Q6: floor of the fp32 parameter times F, evaluated in fp64.
        return int(np.floor(float(np.float32(self.bits_per_value)) * self.F))

    def check(self):
        if self.F <= 0 or self.group <= 0 or self.F % self.group:
            raise OracleError("F must be a positive multiple of the group size")
        if self.group % 8:
            raise OracleError("group size must be a multiple of 8")
        if not 0 <= self.max_bits <= 8:
            raise OracleError("max_bits must be in 0..8")


@dataclasses.dataclass
class Slot:
    """Calibration result for one (layer, kind)."""
    layer: int
    kind: int
    F: int
    G: int
    widths: np.ndarray      # u8 [F/G]
    mu32: np.ndarray        # f32 [F]
    lam: np.ndarray         # f64 [F]
    V32: np.ndarray         # f32 [F, r_eff]  (active columns only)
    # Diagnostics kept by calibrate() (not serialized):
    mu64: np.ndarray | None = None
    V64: np.ndarray | None = None
    D: np.ndarray | None = None
    # Per-component widths (reading Q2c), u8 [F]; None for group widths.
    # With them, widths[g] is the group's largest component width.
    cwidths: np.ndarray | None = None

    @property
    def active_groups(self) -> np.ndarray:
        return np.nonzero(self.widths)[0]

    @property
    def n_act(self) -> int:
        return int(np.count_nonzero(self.widths))

    @property
    def r_eff(self) -> int:
        return self.n_act * self.G

    @property
    def record_bytes(self) -> int:
        if self.cwidths is not None:
            return 8 * self.n_act + sum(chunk_bytes_pc(self.group_cwidths(g)) for g in self.active_groups)
        return 8 * self.n_act + self.G * int(np.sum(self.widths.astype(np.int64))) // 8

    def group_cwidths(self, g: int) -> np.ndarray:
        """Component widths of group g (Q2c)."""
        return self.cwidths[g * self.G:(g + 1) * self.G]

    def basis_bf16(self) -> np.ndarray:
        """Operational basis V' = bf16_rne(V32) over the active columns (N1)."""
        return bf16_rne(self.V32)

    def serialize(self) -> bytes:
        pc = self.cwidths is not None
        n_w = self.F if pc else self.F // self.G
        head = SLOT_MAGIC + struct.pack("<7i", self.layer, self.kind, self.F, self.G,
                                        self.n_act, self.r_eff, 1 if pc else 0)
        w = np.zeros((n_w + 7) // 8 * 8, np.uint8)
        w[:n_w] = self.cwidths if pc else self.widths
        body = (head + w.tobytes() + np.asarray(self.mu32, "<f4").tobytes()
                + np.asarray(self.lam, "<f8").tobytes()
                + np.ascontiguousarray(self.V32, "<f4").tobytes())
        return body + struct.pack("<Q", fnv1a64(body))

    @property
    def slot_id(self) -> int:
        return struct.unpack("<Q", self.serialize()[-8:])[0]


@dataclasses.dataclass
class Artifact:
    params: Params
    slots: dict          # (layer, kind) -> Slot

    def serialize(self) -> bytes:
        p = self.params
        out = [ART_MAGIC, struct.pack("<I7ifii", FORMAT_VERSION, p.n_layers, p.kv_heads,
                                      p.head_dim, p.sink, p.window, p.group, p.max_bits,
                                      p.bits_per_value, p.dtype, len(self.slots))]
        for key in sorted(self.slots):
            out.append(self.slots[key].serialize())
        return b"".join(out)


def parse_artifact(buf: bytes) -> Artifact:
    """Read the artifact format written out in the module docstring."""
    buf = bytes(buf)
    if buf[:4] != ART_MAGIC:
        raise OracleError("bad artifact magic")
    ver, nl, kh, hd, s, w, g, mb, bpv, dt, n_slots = struct.unpack_from("<I7ifii", buf, 4)
    if ver != FORMAT_VERSION:
        raise OracleError("bad artifact version")
    p = Params(nl, kh, hd, s, w, g, mb, bpv, dt)
    p.check()
    off = 4 + 44
    slots = {}
    for _ in range(n_slots):
        start = off
        if buf[off:off + 4] != SLOT_MAGIC:
            raise OracleError("bad slot magic")
        layer, kind, F, G, n_act, r_eff, pc = struct.unpack_from("<7i", buf, off + 4)
        if pc not in (0, 1):
            raise OracleError("bad slot mode")
        off += 32
        n_g = F // G
        n_w = F if pc else n_g
        wpad = (n_w + 7) // 8 * 8
        widths = np.frombuffer(buf, np.uint8, n_w, off).copy()
        cwidths = None
        if pc:
            cwidths = widths
            widths = cwidths.reshape(n_g, G).max(axis=1).astype(np.uint8)
        off += wpad
        mu32 = np.frombuffer(buf, "<f4", F, off).copy()
        off += 4 * F
        lam = np.frombuffer(buf, "<f8", F, off).copy()
        off += 8 * F
        V32 = np.frombuffer(buf, "<f4", F * r_eff, off).copy().reshape(F, r_eff)
        off += 4 * F * r_eff
        (sid,) = struct.unpack_from("<Q", buf, off)
        if fnv1a64(buf[start:off]) != sid:
            raise OracleError("slot id mismatch")
        off += 8
        sl = Slot(layer, kind, F, G, widths, mu32, lam, V32, cwidths=cwidths)
        if sl.n_act != n_act or sl.r_eff != r_eff:
            raise OracleError("inconsistent slot")
        slots[(layer, kind)] = sl
    return Artifact(p, slots)


# ------------------------------------------------------------- quantizer ---

def quantize_fp32(c: np.ndarray, b: int):
    """Microscaled uniform quantizer of one group, fp32 arithmetic (Q1, Q4, N2).

    c: fp32 [T, G] coefficients of one group.  Returns (codes u8 [T, G],
    shift f32 [T], scale f32 [T])."""
    c = np.asarray(c, np.float32)
    k = np.float32(2 ** b - 1)
    shift = c.min(axis=1)
    scale = (c.max(axis=1) - shift).astype(np.float32)
    nz = scale > 0
    inv = np.zeros_like(scale)
    inv[nz] = k / scale[nz]                                  # IEEE fp32 division
    u = ((c - shift[:, None]).astype(np.float32) * inv[:, None]).astype(np.float32)
    q = np.clip(np.rint(u), 0, k)
    q[~nz] = 0
    return q.astype(np.uint8), shift.astype(np.float32), scale


def quantize_fp32_pc(c: np.ndarray, bs):
    """The group quantizer with a width per component (reading Q2c): the
    group's shift and scale over all its components, component j on
    2^bs[j] - 1 levels; a zero width gives code 0."""
    c = np.asarray(c, np.float32)
    shift = c.min(axis=1)
    scale = (c.max(axis=1) - shift).astype(np.float32)
    nz = scale > 0
    q = np.zeros(c.shape, np.uint8)
    d = (c - shift[:, None]).astype(np.float32)
    for j, b in enumerate(bs):
        if b == 0:
            continue
        k = np.float32(2 ** int(b) - 1)
        inv = np.zeros_like(scale)
        inv[nz] = k / scale[nz]                              # IEEE fp32 division
        u = (d[:, j] * inv).astype(np.float32)
        qj = np.clip(np.rint(u), 0, k)
        qj[~nz] = 0
        q[:, j] = qj.astype(np.uint8)
    return q, shift.astype(np.float32), scale


def dequantize_pc(q, shift, scale, bs) -> np.ndarray:
    """Inverse of quantize_fp32_pc in fp64; a zero width decodes to 0."""
    out = np.zeros(q.shape)
    for j, b in enumerate(bs):
        if b:
            out[:, j] = dequantize(q[:, j:j + 1], shift, scale, int(b))[:, 0]
    return out


def quant_dequant_fp64_pc(c: np.ndarray, b: int, j: int) -> np.ndarray:
    """Component j of group rows c [n, G] through b levels of the group's
    fp64 grid (for the distortion table of reading Q2c)."""
    k = float(2 ** b - 1)
    shift = c.min(axis=1)
    scale = c.max(axis=1) - shift
    out = c[:, j].copy()
    nz = scale > 0
    q = np.clip(np.rint((c[nz, j] - shift[nz]) * (k / scale[nz])), 0, k)
    out[nz] = shift[nz] + q * (scale[nz] / k)
    return out


def dequantize(q: np.ndarray, shift: np.ndarray, scale: np.ndarray, b: int) -> np.ndarray:
    """Inverse of quantize_fp32 in fp64: shift + q * fp32(scale / (2^b - 1))."""
    step = (np.asarray(scale, np.float32) / np.float32(2 ** b - 1)).astype(np.float32)
    return (np.asarray(shift, np.float32).astype(np.float64)[:, None]
            + q.astype(np.float64) * step.astype(np.float64)[:, None])


def quant_dequant_fp64(c: np.ndarray, b: int) -> np.ndarray:
    """The same quantizer carried out in fp64, used for the DP's distortion (Q5)."""
    k = float(2 ** b - 1)
    shift = c.min(axis=1, keepdims=True)
    scale = c.max(axis=1, keepdims=True) - shift
    out = c.copy()
    nz = scale[:, 0] > 0
    inv = k / scale[nz]
    q = np.clip(np.rint((c[nz] - shift[nz]) * inv), 0, k)
    out[nz] = shift[nz] + q * (scale[nz] / k)
    return out


# ----------------------------------------------------------- calibration ---

def pca_basis(xc: np.ndarray):
    """Orthonormal PCA basis of centred rows by SVD (section 2A), readings R2.

    Returns (V [F, F] fp64, lambda [F] fp64)."""
    n, F = xc.shape
    _, s, vt = np.linalg.svd(xc, full_matrices=n < F)
    sv = np.zeros(F)
    sv[: s.size] = s
    order = np.argsort(-sv, kind="stable")
    V = vt.T[:, order].copy()
    lam = sv[order] ** 2 / n
    for j in range(F):
        col = V[:, j]
        i = int(np.argmax(np.abs(col)))          # first index among equal maxima
        if col[i] < 0:
            V[:, j] = -col
    return V, lam


def distortion_table(C: np.ndarray, G: int, max_bits: int) -> np.ndarray:
    """D[g, b] = mean over rows of the group's squared quantization error (Q5).

    b = 0 drops the group: its error is the group's energy."""
    n, F = C.shape
    D = np.zeros((F // G, max_bits + 1))
    for g in range(F // G):
        cg = C[:, g * G:(g + 1) * G]
        D[g, 0] = np.mean(np.sum(cg * cg, axis=1))
        for b in range(1, max_bits + 1):
            e = cg - quant_dequant_fp64(cg, b)
            D[g, b] = np.mean(np.sum(e * e, axis=1))
    return D


def group_cost(b: int, G: int) -> int:
    return G * b + (SCALE_BITS if b > 0 else 0)


def dp_allocate(D: np.ndarray, G: int, budget: int) -> np.ndarray:
    """Widths minimising sum_g D[g, b_g] subject to sum_g cost(b_g) <= budget
    (section 2A, dynamic-programming bit allocation; ties by reading Q7).

    f[g][u] = least distortion of groups g.. that spend exactly u bits,
    f[g][u] = min_b D[g, b] + f[g+1][u - cost(b)], evaluated last group first
    so every objective is the nested sum D[0] + (D[1] + (... + 0))."""
    n_g, nb = D.shape
    if budget < 0:
        raise OracleError("negative budget")
    INF = np.inf
    f = np.full((n_g + 1, budget + 1), INF)
    f[n_g, 0] = 0.0
    for g in range(n_g - 1, -1, -1):
        for u in range(budget + 1):
            best = INF
            for b in range(nb):
                c = group_cost(b, G)
                if c <= u and f[g + 1, u - c] < INF:
                    v = D[g, b] + f[g + 1, u - c]
                    if v < best:
                        best = v
            f[g, u] = best
    u = int(np.argmin(f[0]))                  # first minimum = fewest bits
    widths = np.zeros(n_g, np.uint8)
    for g in range(n_g):
        for b in range(nb - 1, -1, -1):        # largest width first
            c = group_cost(b, G)
            if c <= u and D[g, b] + f[g + 1, u - c] == f[g, u]:
                widths[g] = b
                u -= c
                break
        else:
            raise OracleError("DP reconstruction failed")
    return widths


def slot_dp_table(D: np.ndarray, G: int, max_bits_used: int, max_active: int) -> np.ndarray:
    """f[g, u, r] = least distortion of groups g.. of one tensor spending
    exactly u bits with at most r active groups (used by dp_allocate_global).

    Same recurrence and nesting as dp_allocate, f[g][u][r] = min_b D[g, b] +
    f[g+1][u - cost(b)][r - (b > 0)], evaluated for every u at once."""
    n_g, nb = D.shape
    U = max_bits_used
    f = np.full((n_g + 1, U + 1, max_active + 1), np.inf)
    f[n_g, 0, :] = 0.0
    for g in range(n_g - 1, -1, -1):
        for r in range(max_active + 1):
            best = np.full(U + 1, np.inf)
            for b in range(nb):
                c, rr = group_cost(b, G), r - (1 if b > 0 else 0)
                if rr < 0 or c > U:
                    continue
                cand = np.full(U + 1, np.inf)
                cand[c:] = D[g, b] + f[g + 1, : U + 1 - c, rr]
                best = np.minimum(best, cand)
            f[g, :, r] = best
    return f


def distortion_table_pc(C: np.ndarray, G: int, max_bits: int) -> np.ndarray:
    """Dc[j, b] = mean over rows of component j's squared error at b bits on
    its group's grid (reading Q2c); b = 0 drops it (its energy)."""
    n, F = C.shape
    Dc = np.zeros((F, max_bits + 1))
    for g in range(F // G):
        cg = C[:, g * G:(g + 1) * G]
        for j in range(G):
            Dc[g * G + j, 0] = np.mean(cg[:, j] ** 2)
            for b in range(1, max_bits + 1):
                e = cg[:, j] - quant_dequant_fp64_pc(cg, b, j)
                Dc[g * G + j, b] = np.mean(e * e)
    return Dc


def chunk_bytes_pc(bs) -> int:
    return (int(np.sum(np.asarray(bs, np.int64))) + 7) // 8


def group_cost_pc(s: int) -> int:
    """Bits of a group whose component widths sum to s (reading Q2c)."""
    return 0 if s == 0 else SCALE_BITS + 8 * ((s + 7) // 8)


def _pc_inner(Dc: np.ndarray, G: int):
    """Per group g, e[i][s] = least distortion of components i.. of the group
    whose widths sum to s (nested from the last component)."""
    F, nb = Dc.shape
    n_g = F // G
    smax = (nb - 1) * G
    INF = np.inf
    inner = []
    for g in range(n_g):
        D = Dc[g * G:(g + 1) * G]
        e = np.full((G + 1, smax + 1), INF)
        e[G, 0] = 0.0
        for i in range(G - 1, -1, -1):
            for sm in range(smax + 1):
                best = INF
                for b in range(nb):
                    if b <= sm and e[i + 1, sm - b] < INF:
                        v = D[i, b] + e[i + 1, sm - b]
                        if v < best:
                            best = v
                e[i, sm] = best
        inner.append(e)
    return inner


def _pc_components(Dc: np.ndarray, G: int, g: int, e: np.ndarray, sm: int, out: np.ndarray):
    """Group g's component widths summing to sm, largest width first."""
    nb = Dc.shape[1]
    D = Dc[g * G:(g + 1) * G]
    for i in range(G):
        for b in range(min(nb - 1, sm), -1, -1):
            if e[i + 1, sm - b] < np.inf and D[i, b] + e[i + 1, sm - b] == e[i, sm]:
                out[g * G + i] = b
                sm -= b
                break
        else:
            raise OracleError("DP reconstruction failed (component)")


def dp_allocate_pc(Dc: np.ndarray, G: int, budget: int, max_active: int | None = None) -> np.ndarray:
    """Component widths minimising sum_j Dc[j, b_j] within the budget, with
    the cost of reading Q2c (ties in its order); with max_active, at most
    that many active groups (reading Q3c: the plain result whenever it keeps
    to the cap, else _dp_allocate_pc_capped's).

    Per group, e[i][s] (see _pc_inner); across groups,
    f[g][u] = min_s E_g(s) + f[g+1][u - cost(s)] (nested from the last)."""
    out = _dp_allocate_pc_plain(Dc, G, budget)
    if max_active is not None and np.count_nonzero(out.reshape(-1, G).sum(axis=1)) > max_active:
        out = _dp_allocate_pc_capped(Dc, G, budget, max_active)
    return out


def _dp_allocate_pc_capped(Dc: np.ndarray, G: int, budget: int, max_active: int) -> np.ndarray:
    """The allocation of dp_allocate_pc with at most max_active active groups:
    f[g][u][r] = least distortion of groups g.. at exactly u bits with at
    most r of them active, f[g][u][r] = min(f[g+1][u][r], min_{s>0} E_g(s) +
    f[g+1][u - cost(s)][r - 1]); the same tie order (fewest bits, then the
    largest sum for the earliest group, then the largest widths first)."""
    F, nb = Dc.shape
    n_g = F // G
    smax = (nb - 1) * G
    INF = np.inf
    inner = _pc_inner(Dc, G)
    R = max_active
    f = np.full((n_g + 1, budget + 1, R + 1), INF)
    f[n_g, 0, :] = 0.0
    for g in range(n_g - 1, -1, -1):
        for r in range(R + 1):
            best = np.full(budget + 1, INF)       # over u at once
            for sm in range(smax + 1):
                c = group_cost_pc(sm)
                rr = r - (1 if sm > 0 else 0)
                if c <= budget and rr >= 0 and inner[g][0, sm] < INF:
                    best[c:] = np.minimum(best[c:], inner[g][0, sm] + f[g + 1, :budget + 1 - c, rr])
            f[g, :, r] = best
    u = int(np.argmin(f[0, :, R]))               # first minimum = fewest bits
    r = R
    out = np.zeros(F, np.uint8)
    for g in range(n_g):
        e = inner[g]
        for sm in range(smax, -1, -1):            # largest sum first
            c = group_cost_pc(sm)
            rr = r - (1 if sm > 0 else 0)
            if c <= u and rr >= 0 and e[0, sm] < INF and e[0, sm] + f[g + 1, u - c, rr] == f[g, u, r]:
                break
        else:
            raise OracleError("DP reconstruction failed (group)")
        u -= c
        r = rr
        _pc_components(Dc, G, g, e, sm, out)
    return out


def _dp_allocate_pc_plain(Dc: np.ndarray, G: int, budget: int) -> np.ndarray:
    F, nb = Dc.shape
    n_g = F // G
    smax = (nb - 1) * G
    INF = np.inf
    inner = _pc_inner(Dc, G)
    f = np.full((n_g + 1, budget + 1), INF)
    f[n_g, 0] = 0.0
    for g in range(n_g - 1, -1, -1):
        for u in range(budget + 1):
            best = INF
            for sm in range(smax + 1):
                c = group_cost_pc(sm)
                if c <= u and inner[g][0, sm] < INF and f[g + 1, u - c] < INF:
                    v = inner[g][0, sm] + f[g + 1, u - c]
                    if v < best:
                        best = v
            f[g, u] = best
    u = int(np.argmin(f[0]))                  # first minimum = fewest bits
    out = np.zeros(F, np.uint8)
    for g in range(n_g):
        e = inner[g]
        for sm in range(smax, -1, -1):        # largest sum first
            c = group_cost_pc(sm)
            if c <= u and e[0, sm] < INF and e[0, sm] + f[g + 1, u - c] == f[g, u]:
                break
        else:
            raise OracleError("DP reconstruction failed (group)")
        u -= c
        _pc_components(Dc, G, g, e, sm, out)
    return out


def dp_allocate_global(Ds, G: int, budget_per_tensor: int, max_active: int):
    """Widths of several tensors chosen together (readings Q6g, Q7g).

    Ds: the distortion tables D[g, b] of the tensors, in (layer, kind) order.
    Minimises sum_s sum_g D_s[g, b_sg] subject to sum_s sum_g cost(b_sg) <=
    len(Ds) * budget_per_tensor and at most max_active active groups per
    tensor.  e_s[u] = f_s[0, u, max_active] is tensor s's least distortion at
    exactly u bits; H[s][U] = min_u e_s[u] + H[s+1][U - u] combines them."""
    S = len(Ds)
    B = S * budget_per_tensor
    if budget_per_tensor < 0 or max_active < 0:
        raise OracleError("negative budget or cap")
    tables, es = [], []
    for D in Ds:
        n_g, nb = D.shape
        top = min(B, min(n_g, max_active) * group_cost(nb - 1, G))
        f = slot_dp_table(D, G, top, max_active)
        tables.append(f)
        es.append(f[0, :, max_active])
    H = np.full((S + 1, B + 1), np.inf)
    H[S, 0] = 0.0
    for s in range(S - 1, -1, -1):
        for u, e in enumerate(es[s]):
            if e < np.inf:
                H[s, u:] = np.minimum(H[s, u:], e + H[s + 1, : B + 1 - u])
    U = int(np.argmin(H[0]))                   # first minimum = fewest bits
    out = []
    for s in range(S):
        e, f, D = es[s], tables[s], Ds[s]
        for u in range(min(U, e.size - 1), -1, -1):      # most bits to the earlier tensor
            if e[u] < np.inf and e[u] + H[s + 1, U - u] == H[s, U]:
                break
        else:
            raise OracleError("global DP reconstruction failed (tensor level)")
        U -= u
        n_g, nb = D.shape
        w = np.zeros(n_g, np.uint8)
        r = max_active
        for g in range(n_g):
            for b in range(nb - 1, -1, -1):              # largest width first (Q7)
                c, rr = group_cost(b, G), r - (1 if b > 0 else 0)
                if c <= u and rr >= 0 and D[g, b] + f[g + 1, u - c, rr] == f[g, u, r]:
                    w[g] = b
                    u, r = u - c, rr
                    break
            else:
                raise OracleError("global DP reconstruction failed (group level)")
        out.append(w)
    return out


def shared_pca(rows_list):
    """One basis for several tensors (reading P1s): every tensor's rows are
    centred on that tensor's own mean, then pooled, then pca_basis."""
    return pca_basis(np.vstack([r - r.mean(axis=0) for r in rows_list]))


def _make_slot(layer, kind, params: Params, mu, V, lam, D, widths) -> Slot:
    G = params.group
    cols = np.concatenate([np.arange(g * G, (g + 1) * G) for g in np.nonzero(widths)[0]]
                          ) if np.any(widths) else np.zeros(0, np.int64)
    return Slot(layer, kind, params.F, G, np.asarray(widths, np.uint8), mu.astype(np.float32),
                lam, V[:, cols].astype(np.float32), mu64=mu, V64=V, D=D)


def calibrate_set(inputs, params: Params, shared_basis: bool = False,
                  global_budget: bool = False, max_active: int | None = None,
                  component_widths: bool = False) -> dict:
    """Calibrate several tensors at once (readings P1s, Q6g, Q7g).

    inputs: (layer, kind, x_cal [n, F]) triples, at most one per (layer, kind).
    shared_basis: one PCA basis per kind over the pooled rows of its tensors,
    each centred on its own mean.  global_budget: widths from
    dp_allocate_global with at most max_active active groups per tensor (no cap
    if None).  component_widths: a width per component (reading Q2c), with at
    most max_active active groups when given (reading Q3c).  Without a flag
    every tensor is calibrate()'s result.
    Returns {(layer, kind): Slot}."""
    params.check()
    prep = {}
    for layer, kind, x_cal in inputs:
        x = np.asarray(x_cal, np.float64)
        n, F = x.shape
        if F != params.F:
            raise OracleError("feature count mismatch")
        if (layer, kind) in prep:
            raise OracleError("a (layer, kind) appears twice")
        rows = x[params.sink: n - params.window]                 # R1
        if rows.shape[0] < 1:
            raise OracleError("no calibration rows after sink and window")
        prep[(layer, kind)] = rows
    keys = sorted(prep)
    mus = {k: prep[k].mean(axis=0) for k in keys}
    basis = {}
    if shared_basis:
        for kind in sorted({k for _, k in keys}):
            same = [key for key in keys if key[1] == kind]
            Vl = shared_pca([prep[key] for key in same])
            for key in same:
                basis[key] = Vl
    else:
        for key in keys:
            basis[key] = pca_basis(prep[key] - mus[key])
    if component_widths:
        if global_budget:
            raise OracleError("component widths take a budget per tensor")
        out = {}
        for k in keys:
            C = (prep[k] - mus[k]) @ basis[k][0]
            Dc = distortion_table_pc(C, params.group, params.max_bits)
            cw = dp_allocate_pc(Dc, params.group, params.budget_bits, max_active)
            widths = cw.reshape(-1, params.group).max(axis=1).astype(np.uint8)
            sl = _make_slot(k[0], k[1], params, mus[k], basis[k][0], basis[k][1], Dc, widths)
            sl.cwidths = cw
            out[k] = sl
        return out
    D = {key: distortion_table((prep[key] - mus[key]) @ basis[key][0], params.group,
                               params.max_bits) for key in keys}
    if global_budget:
        cap = params.n_groups if max_active is None else max_active
        ws = dict(zip(keys, dp_allocate_global([D[k] for k in keys], params.group,
                                               params.budget_bits, cap)))
    elif max_active is None:
        ws = {k: dp_allocate(D[k], params.group, params.budget_bits) for k in keys}
    else:
        ws = {k: dp_allocate_global([D[k]], params.group, params.budget_bits, max_active)[0]
              for k in keys}
    return {k: _make_slot(k[0], k[1], params, mus[k], basis[k][0], basis[k][1], D[k], ws[k])
            for k in keys}


def calibrate(x_cal: np.ndarray, params: Params, layer: int, kind: int,
              max_active: int | None = None) -> Slot:
    """Calibrate one (layer, kind) from calibration rows x_cal [n, F] (values).

    max_active: at most this many active groups (the widths then minimise the
    distortion under both the budget and the cap: dp_allocate_global of the
    one tensor, which is dp_allocate whenever the cap does not bind)."""
    params.check()
    x = np.asarray(x_cal, np.float64)
    n, F = x.shape
    if F != params.F:
        raise OracleError("feature count mismatch")
    rows = x[params.sink: n - params.window]                     # R1
    if rows.shape[0] < 1:
        raise OracleError("no calibration rows after sink and window")
    mu = rows.mean(axis=0)
    xc = rows - mu
    V, lam = pca_basis(xc)
    C = xc @ V
    D = distortion_table(C, params.group, params.max_bits)
    if max_active is None:
        widths = dp_allocate(D, params.group, params.budget_bits)
    else:
        (widths,) = dp_allocate_global([D], params.group, params.budget_bits, max_active)
    G = params.group
    cols = np.concatenate([np.arange(g * G, (g + 1) * G) for g in np.nonzero(widths)[0]]
                          ) if np.any(widths) else np.zeros(0, np.int64)
    return Slot(layer, kind, F, G, widths, mu.astype(np.float32), lam,
                V[:, cols].astype(np.float32), mu64=mu, V64=V, D=D)


# ------------------------------------------------------------------ stream ---

def split_rows(T: int, s: int, w: int):
    """Effective sink and window (reading W1): s' = min(s, T), w' = min(w, T - s')."""
    s1 = min(s, T)
    w1 = min(w, T - s1)
    return s1, w1, T - s1 - w1


def pack_codes(q: np.ndarray, b: int) -> np.ndarray:
    """Codes [T, G] of width b -> bytes [T, G*b/8], LSB-first."""
    T, G = q.shape
    bits = ((q.astype(np.uint16)[:, :, None] >> np.arange(b, dtype=np.uint16)) & 1)
    return np.packbits(bits.astype(np.uint8).reshape(T, G * b), axis=1, bitorder="little")


def pack_codes_pc(q: np.ndarray, bs) -> np.ndarray:
    """Codes [T, G] with a width per component -> bytes [T, ceil(sum b / 8)]:
    code j at bit sum_{i<j} b_i, LSB first, zero padded (reading Q2c)."""
    T = q.shape[0]
    cols = [((q[:, j].astype(np.uint16)[:, None] >> np.arange(int(b), dtype=np.uint16)) & 1)
            for j, b in enumerate(bs) if b]
    nbits = int(np.sum(np.asarray(bs, np.int64)))
    bits = np.zeros((T, chunk_bytes_pc(bs) * 8), np.uint8)
    if cols:
        bits[:, :nbits] = np.concatenate(cols, axis=1)
    return np.packbits(bits, axis=1, bitorder="little")


def unpack_codes_pc(chunk: np.ndarray, bs) -> np.ndarray:
    T = chunk.shape[0]
    bits = np.unpackbits(chunk, axis=1, bitorder="little")
    q = np.zeros((T, len(bs)), np.uint8)
    pos = 0
    for j, b in enumerate(bs):
        b = int(b)
        if b:
            q[:, j] = np.sum(bits[:, pos:pos + b].astype(np.uint16) << np.arange(b, dtype=np.uint16),
                             axis=1).astype(np.uint8)
        pos += b
    return q


def unpack_codes(chunk: np.ndarray, G: int, b: int) -> np.ndarray:
    T = chunk.shape[0]
    bits = np.unpackbits(chunk, axis=1, bitorder="little").reshape(T, G, b)
    return np.sum(bits.astype(np.uint16) << np.arange(b, dtype=np.uint16), axis=2).astype(np.uint8)


def make_header(params: Params, slot: Slot, layer: int, kind: int, T: int) -> bytes:
    s1, w1, tc = split_rows(T, params.sink, params.window)
    h = STREAM_MAGIC + struct.pack("<HBBIIIIIIHHIQ", FORMAT_VERSION, params.dtype, kind,
                                   layer, T, params.F, s1, w1, tc, slot.G, slot.n_act,
                                   slot.record_bytes, slot.slot_id)
    return h + bytes(HEADER_BYTES - len(h))


def stream_bytes(params: Params, slot: Slot, T: int) -> int:
    s1, w1, tc = split_rows(T, params.sink, params.window)
    return HEADER_BYTES + (s1 + w1) * params.F * params.elem_bytes + tc * slot.record_bytes


def _values(x_store: np.ndarray, dtype: int) -> np.ndarray:
    return bf16_to_f32(x_store) if dtype == DTYPE_BF16 else np.asarray(x_store, np.float32)


@dataclasses.dataclass
class EncodeResult:
    stream: bytes
    codes: np.ndarray        # u8 [T_c, r_eff]
    shift: np.ndarray        # f32 [T_c, n_act]
    scale: np.ndarray        # f32 [T_c, n_act]
    coeffs: np.ndarray       # f32 [T_c, r_eff]


def project(x_vals: np.ndarray, slot: Slot) -> np.ndarray:
    """Centre and project (section 2B): c = fp32(sum_f (x_f - mu32_f) V'_fj), fp64 (N1)."""
    xc = x_vals.astype(np.float64) - slot.mu32.astype(np.float64)
    return (xc @ slot.basis_bf16().astype(np.float64)).astype(np.float32)


def build_records(codes, shift, scale, slot: Slot) -> np.ndarray:
    tc = codes.shape[0]
    parts = []
    ss = np.empty((tc, slot.n_act, 2), "<f4")
    ss[:, :, 0] = shift
    ss[:, :, 1] = scale
    parts.append(ss.view(np.uint8).reshape(tc, 8 * slot.n_act))
    for a, g in enumerate(slot.active_groups):
        q = codes[:, a * slot.G:(a + 1) * slot.G]
        if slot.cwidths is not None:
            parts.append(pack_codes_pc(q, slot.group_cwidths(g)))
        else:
            parts.append(pack_codes(q, int(slot.widths[g])))
    if not parts or tc == 0:
        return np.zeros((tc, slot.record_bytes), np.uint8)
    return np.concatenate(parts, axis=1)


def encode(x_store: np.ndarray, params: Params, slot: Slot, layer: int, kind: int) -> EncodeResult:
    """Compress one [T, F] tensor given as raw element storage (uint16 bf16 or f32)."""
    T, F = x_store.shape
    if F != params.F:
        raise OracleError("feature count mismatch")
    s1, w1, tc = split_rows(T, params.sink, params.window)
    raw = np.ascontiguousarray(x_store)
    passthrough = np.concatenate([raw[:s1], raw[T - w1:]], axis=0)
    x = _values(raw[s1:T - w1], params.dtype)
    c = project(x, slot) if slot.r_eff else np.zeros((tc, 0), np.float32)
    codes = np.zeros((tc, slot.r_eff), np.uint8)
    shift = np.zeros((tc, slot.n_act), np.float32)
    scale = np.zeros((tc, slot.n_act), np.float32)
    for a, g in enumerate(slot.active_groups):
        sl = slice(a * slot.G, (a + 1) * slot.G)
        if slot.cwidths is not None:
            codes[:, sl], shift[:, a], scale[:, a] = quantize_fp32_pc(c[:, sl], slot.group_cwidths(g))
        else:
            codes[:, sl], shift[:, a], scale[:, a] = quantize_fp32(c[:, sl], int(slot.widths[g]))
    rec = build_records(codes, shift, scale, slot)
    stream = (make_header(params, slot, layer, kind, T) + passthrough.tobytes()
              + rec.tobytes())
    return EncodeResult(stream, codes, shift, scale, c)


@dataclasses.dataclass
class Header:
    version: int
    dtype: int
    kind: int
    layer: int
    T: int
    F: int
    s: int
    w: int
    tc: int
    G: int
    n_act: int
    record_bytes: int
    slot_id: int


def parse_header(stream: bytes) -> Header:
    if len(stream) < HEADER_BYTES or stream[:4] != STREAM_MAGIC:
        raise OracleError("bad stream magic")
    return Header(*struct.unpack_from("<HBBIIIIIIHHIQ", stream, 4))


def check_header(h: Header, params: Params, slot: Slot, layer: int, kind: int, T: int):
    s1, w1, tc = split_rows(T, params.sink, params.window)
    want = Header(FORMAT_VERSION, params.dtype, kind, layer, T, params.F, s1, w1, tc,
                  slot.G, slot.n_act, slot.record_bytes, slot.slot_id)
    if h != want:
        raise OracleError(f"stream header mismatch: {h} != {want}")


def read_records(stream: bytes, params: Params, slot: Slot, T: int):
    """Records -> (codes u8 [T_c, r_eff], shift f32 [T_c, n_act], scale f32)."""
    s1, w1, tc = split_rows(T, params.sink, params.window)
    off = HEADER_BYTES + (s1 + w1) * params.F * params.elem_bytes
    rb = slot.record_bytes
    rec = np.frombuffer(stream, np.uint8, tc * rb, off).reshape(tc, rb)
    ss = rec[:, :8 * slot.n_act].copy().view("<f4").reshape(tc, slot.n_act, 2)
    codes = np.zeros((tc, slot.r_eff), np.uint8)
    pos = 8 * slot.n_act
    for a, g in enumerate(slot.active_groups):
        if slot.cwidths is not None:
            bs = slot.group_cwidths(g)
            nbytes = chunk_bytes_pc(bs)
            codes[:, a * slot.G:(a + 1) * slot.G] = unpack_codes_pc(rec[:, pos:pos + nbytes], bs)
        else:
            b = int(slot.widths[g])
            nbytes = slot.G * b // 8
            codes[:, a * slot.G:(a + 1) * slot.G] = unpack_codes(rec[:, pos:pos + nbytes], slot.G, b)
        pos += nbytes
    return codes, ss[:, :, 0].astype(np.float32), ss[:, :, 1].astype(np.float32)


def reconstruct(codes, shift, scale, slot: Slot) -> np.ndarray:
    """Dequantize, multiply by V'^T, add the mean (section 2C); fp64 [T_c, F]."""
    tc = codes.shape[0]
    chat = np.zeros((tc, slot.r_eff))
    for a, g in enumerate(slot.active_groups):
        sl = slice(a * slot.G, (a + 1) * slot.G)
        if slot.cwidths is not None:
            chat[:, sl] = dequantize_pc(codes[:, sl], shift[:, a], scale[:, a], slot.group_cwidths(g))
        else:
            chat[:, sl] = dequantize(codes[:, sl], shift[:, a], scale[:, a], int(slot.widths[g]))
    return slot.mu32.astype(np.float64) + chat @ slot.basis_bf16().astype(np.float64).T


def decode(stream: bytes, params: Params, slot: Slot, layer: int, kind: int, T: int,
           out_dtype: int = DTYPE_F32):
    """Decompress one stream.  Returns (x_hat fp64 [T, F], out storage [T, F]).

    Passthrough rows come back verbatim (converted if out_dtype differs)."""
    stream = bytes(stream)
    h = parse_header(stream)
    check_header(h, params, slot, layer, kind, T)
    F = params.F
    s1, w1, tc = h.s, h.w, h.tc
    if len(stream) < stream_bytes(params, slot, T):
        raise OracleError("truncated stream")
    sdt = np.uint16 if params.dtype == DTYPE_BF16 else np.float32
    pt = np.frombuffer(stream, sdt, (s1 + w1) * F, HEADER_BYTES).reshape(s1 + w1, F)
    pt_vals = _values(pt, params.dtype).astype(np.float64)
    codes, shift, scale = read_records(stream, params, slot, T)
    xh = reconstruct(codes, shift, scale, slot) if tc else np.zeros((0, F))
    full = np.concatenate([pt_vals[:s1], xh, pt_vals[s1:]], axis=0)
    if out_dtype == params.dtype:
        store_pt = pt
    elif out_dtype == DTYPE_BF16:
        store_pt = f32_to_bf16_bits(pt_vals.astype(np.float32))
    else:
        store_pt = pt_vals.astype(np.float32)
    if out_dtype == DTYPE_BF16:
        body = f32_to_bf16_bits(xh.astype(np.float32))
    else:
        body = xh.astype(np.float32)
    out = np.concatenate([store_pt[:s1], body, store_pt[s1:]], axis=0)
    return full, out


def deflate_ratio(stream: bytes, raw_bytes: int):
    """DEFLATE stage (section 2B), here zlib level 6, for the ratio only (Z1).

    Returns (raw / stream bytes, raw / deflated bytes, the deflated bytes)."""
    z = zlib.compress(bytes(stream), 6)
    return raw_bytes / len(stream), raw_bytes / len(z), z
