"""Plain CPU oracle of the lossless stage that follows KVTC's bit packing.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke entry point and by
the CPU-baseline leg of the benchmark.  The HIP library never imports, links or
calls anything here and shares no code with it; the two meet only through the
container format written out below.

Source: the page "KV Cache Transform Coding for Compact Storage in LLM
Inference" (gist.science, paper 2511.01815), section 2B: after packing, the
integers go through DEFLATE, which the paper runs on the GPU with nvCOMP.  The
pages fix no lossless coder.  This stage replaces that step with a coder of
our own that knows the stream's layout (READING L1):

  L1  A KVTC stream is split into fields, each a sequence of symbols of one
      kind: the byte planes of the passthrough elements, the byte planes of
      the fp32 shifts and of the fp32 scales, and the codes of each active
      group (one symbol per code, alphabet 2^b).  Each field is coded on its
      own with a static model (its normalised histogram) by range asymmetric
      numeral systems (rANS: J. Duda, "Asymmetric numeral systems", 2009 and
      2013), in independent chunks of CHUNK symbols with 64 interleaved states each,
      so that chunks code in parallel and the 64 lanes of a wavefront code
      one chunk together.  The 64-byte stream header is kept verbatim.

Fields, in order (esz = 2 for bf16, 4 for f32; n_act active groups):
  P_j, j < esz   byte j (little-endian) of every passthrough element: rows
                 [0, s') then [T - w', T), features in order; alphabet 256
  S_j, j < 4     byte j of every record's fp32 shifts, token-major then group
  R_j, j < 4     the same for the fp32 scales
  Q_a, a < n_act codes of active group a, token-major then component; alphabet
                 2^b_a
A field with no symbols has no chunks and an all-zero table.

With a width per component (reading Q2c of the oracle) the fields are the
same (READING L1c): Q_a still holds all G codes of each record's group a,
component j's code read from its own b_j bits of the group's chunk (a
component of width 0 gives the symbol 0), and its alphabet is 2^b_a with b_a
the group's largest component width; the merge packs each code back into
its own b_j bits, the chunk's padding bits zero.

Model: h = the field's histogram over its alphabet, N = sum h, n_p = number
of symbols present, M = 4096.  f_s = 0 if h_s = 0, else 1 + floor(h_s *
(M - n_p) / N); the remainder M - sum f goes to the most frequent symbol
(lowest index on ties).  c_s = sum of f over symbols below s.

rANS (32-bit states, L = 2^16, 16-bit words), 64 states per chunk: symbol i
of a chunk of n <= CHUNK = 16384 symbols belongs to state (lane) i mod 64 and
to step i div 64.  Encoding starts every state at L and runs the steps from
the last to the first; in a step, every lane with a symbol s: if
x >= f_s * 2^20 it emits the low 16 bits of x and x >>= 16, then
x = floor(x / f_s) * M + (x mod f_s) + c_s.  The chunk's payload is the 64
final states, each as (low word, high word), then the emitted words step by
step from step 0 to the last, inside a step in ascending lane order.
Decoding reads the 64 states and runs the steps from the first: every lane
with a symbol takes slot = x mod M, s with c_s <= slot < c_s + f_s,
x = f_s * floor(x / M) + slot - c_s; then the lanes with x < L, in ascending
lane order, each take the next word w: x = x * 2^16 + w.  Every state ends at
L and every word is used.  (Independent states let the 64 lanes of a GPU
wavefront code one chunk together; the word order is what a wavefront
produces with a ballot and a prefix count.)

Container (little-endian):
  0    "KVTZ", u16 version = 1, u16 n_fields, u32 CHUNK, u32 n_chunks,
       u64 stream_bytes, u64 container_bytes, u32 payload_offset, zeros to 64
  64   the stream's 64-byte header
  128  per field: u32 n_symbols, u16 alphabet A, u16 0, u16 f[A]
  then u32 end[n_chunks]: end of each chunk's payload relative to
       payload_offset (chunks in field order, then chunk order)
  payload_offset = that position rounded up to 16; then the payloads, then
  zeros up to container_bytes, the end of the last payload rounded up to 16
  (so a reader may fetch whole 16-byte blocks).
"""
from __future__ import annotations

import struct

import numpy as np

from .kvtc_oracle import (HEADER_BYTES, OracleError, chunk_bytes_pc, pack_codes, pack_codes_pc, split_rows,
                          unpack_codes, unpack_codes_pc)

MAGIC = b"KVTZ"
VERSION = 1
LANES = 64
CHUNK = 16384
M_BITS = 12
M = 1 << M_BITS
RANS_L = 1 << 16
CONTAINER_HEADER = 64


# ------------------------------------------------------------------ fields ---

def stream_fields(stream: bytes, params, slot, T: int):
    """Split a KVTC stream into its fields (readings L1, L1c): [(symbols u8, A)]."""
    pc = getattr(slot, "cwidths", None) is not None
    s1, w1, tc = split_rows(T, params.sink, params.window)
    esz, F = params.elem_bytes, params.F
    n_pt = (s1 + w1) * F
    buf = np.frombuffer(stream, np.uint8)
    pt = buf[HEADER_BYTES:HEADER_BYTES + n_pt * esz].reshape(n_pt, esz)
    fields = [(pt[:, j].copy(), 256) for j in range(esz)]
    off = HEADER_BYTES + n_pt * esz
    rb, na = slot.record_bytes, slot.n_act
    rec = buf[off:off + tc * rb].reshape(tc, rb)
    ss = rec[:, :8 * na].reshape(tc, na, 2, 4)
    fields += [(ss[:, :, 0, j].reshape(-1).copy(), 256) for j in range(4)]
    fields += [(ss[:, :, 1, j].reshape(-1).copy(), 256) for j in range(4)]
    pos = 8 * na
    for g in slot.active_groups:
        b = int(slot.widths[g])
        if pc:
            bs = slot.group_cwidths(g)
            nbytes = chunk_bytes_pc(bs)
            q = unpack_codes_pc(rec[:, pos:pos + nbytes], bs)
        else:
            nbytes = slot.G * b // 8
            q = unpack_codes(rec[:, pos:pos + nbytes], slot.G, b)
        fields.append((q.reshape(-1).copy(), 1 << b))
        pos += nbytes
    return fields


def merge_fields(header: bytes, fields, params, slot, T: int) -> bytes:
    """Inverse of stream_fields."""
    s1, w1, tc = split_rows(T, params.sink, params.window)
    esz, F = params.elem_bytes, params.F
    n_pt = (s1 + w1) * F
    pt = np.zeros((n_pt, esz), np.uint8)
    for j in range(esz):
        pt[:, j] = fields[j][0]
    na = slot.n_act
    ss = np.zeros((tc, na, 2, 4), np.uint8)
    for j in range(4):
        ss[:, :, 0, j] = fields[esz + j][0].reshape(tc, na)
        ss[:, :, 1, j] = fields[esz + 4 + j][0].reshape(tc, na)
    parts = [ss.reshape(tc, 8 * na)]
    pc = getattr(slot, "cwidths", None) is not None
    for a, g in enumerate(slot.active_groups):
        q = fields[esz + 8 + a][0].reshape(tc, slot.G)
        if pc:
            parts.append(pack_codes_pc(q, slot.group_cwidths(g)))
        else:
            parts.append(pack_codes(q, int(slot.widths[g])))
    rec = np.concatenate(parts, axis=1) if parts else np.zeros((tc, 0), np.uint8)
    return bytes(header) + pt.tobytes() + rec.tobytes()


# ------------------------------------------------------------------- model ---

def normalize(hist: np.ndarray) -> np.ndarray:
    """Frequencies summing to M, every present symbol at least 1 (see header)."""
    h = np.asarray(hist, np.int64)
    N = int(h.sum())
    f = np.zeros(h.size, np.int64)
    if N == 0:
        return f
    present = h > 0
    n_p = int(np.count_nonzero(present))
    f[present] = 1 + (h[present] * (M - n_p)) // N
    f[int(np.argmax(h))] += M - int(f.sum())
    return f


# -------------------------------------------------------------------- rANS ---

def rans_encode(chunks, f: np.ndarray):
    """Encode each chunk (u8 symbol arrays) with frequencies f; returns the
    payloads (u16 word arrays, decoder order).  The 64 lanes of a step are
    computed together."""
    f = np.asarray(f, np.uint64)
    c = np.concatenate([[0], np.cumsum(f)[:-1]]).astype(np.uint64)
    out = []
    for ch in chunks:
        n = len(ch)
        steps = (n + LANES - 1) // LANES
        sym = np.zeros(steps * LANES, np.int64)
        sym[:n] = ch
        x = np.full(LANES, RANS_L, np.uint64)
        groups = []
        for t in range(steps - 1, -1, -1):
            act = np.arange(t * LANES, (t + 1) * LANES) < n
            s = sym[t * LANES:(t + 1) * LANES]
            fs = np.where(act, f[s], 1).astype(np.uint64)     # lanes without a symbol: any f
            emit = act & (x >= (fs << np.uint64(20)))
            groups.append((x[emit] & np.uint64(0xFFFF)).astype(np.uint16))
            x = np.where(emit, x >> np.uint64(16), x)
            x = np.where(act, (x // fs) * np.uint64(M) + (x % fs) + c[s], x)
        states = np.stack([x & np.uint64(0xFFFF), x >> np.uint64(16)], axis=1).reshape(-1)
        out.append(np.concatenate([states.astype(np.uint16)] + groups[::-1]).astype(np.uint16))
    return out


def rans_decode(payloads, lens, f: np.ndarray):
    """Decode each payload into lens[k] symbols."""
    f = np.asarray(f, np.int64)
    c = np.concatenate([[0], np.cumsum(f)[:-1]])
    slot_sym = np.repeat(np.arange(f.size), f)           # slot -> symbol
    out = []
    for words, n in zip(payloads, lens):
        w = np.asarray(words, np.int64)
        if len(w) < 2 * LANES:
            raise OracleError("chunk payload shorter than its states")
        x = w[0:2 * LANES:2] | (w[1:2 * LANES:2] << 16)
        pos = 2 * LANES
        syms = np.zeros(n, np.uint8)
        for t in range((n + LANES - 1) // LANES):
            lanes = np.arange(min(LANES, n - t * LANES))
            slot = x[lanes] & (M - 1)
            s = slot_sym[slot]
            syms[t * LANES + lanes] = s
            x[lanes] = f[s] * (x[lanes] >> M_BITS) + slot - c[s]
            need = lanes[x[lanes] < RANS_L]                    # ascending lanes
            if pos + len(need) > len(w):
                raise OracleError("chunk payload ends early")
            x[need] = (x[need] << 16) | w[pos:pos + len(need)]
            pos += len(need)
        if pos != len(w) or np.any(x != RANS_L):
            raise OracleError("chunk payload does not end at the initial states")
        out.append(syms)
    return out


# --------------------------------------------------------------- container ---

def _chunks(sym):
    return [sym[i:i + CHUNK] for i in range(0, len(sym), CHUNK)]


def compress(stream: bytes, params, slot, T: int) -> bytes:
    """KVTC stream -> KVTZ container (format in the module docstring)."""
    fields = stream_fields(stream, params, slot, T)
    tables, payloads = [], []
    for sym, A in fields:
        f = normalize(np.bincount(sym, minlength=A)) if len(sym) else np.zeros(A, np.int64)
        tables.append(struct.pack("<IHH", len(sym), A, 0) + f.astype("<u2").tobytes())
        payloads += rans_encode(_chunks(sym), f)
    n_chunks = len(payloads)
    ends = np.cumsum([2 * len(p) for p in payloads]).astype("<u4")
    dir_off = CONTAINER_HEADER + HEADER_BYTES + sum(len(t) for t in tables)
    pay_off = (dir_off + 4 * n_chunks + 15) // 16 * 16
    total = (pay_off + (int(ends[-1]) if n_chunks else 0) + 15) // 16 * 16
    head = (MAGIC + struct.pack("<HHIIQQI", VERSION, len(fields), CHUNK, n_chunks, len(stream),
                                total, pay_off))
    body = (head + bytes(CONTAINER_HEADER - len(head)) + bytes(stream[:HEADER_BYTES])
            + b"".join(tables) + ends.tobytes())
    body += bytes(pay_off - len(body))
    body += b"".join(p.astype("<u2").tobytes() for p in payloads)
    body += bytes(total - len(body))
    assert len(body) == total
    return body


def decompress(container: bytes, params, slot, T: int) -> bytes:
    """KVTZ container -> the KVTC stream it holds."""
    buf = bytes(container)
    if buf[:4] != MAGIC:
        raise OracleError("bad container magic")
    ver, n_fields, chunk, n_chunks, stream_bytes, total, pay_off = struct.unpack_from(
        "<HHIIQQI", buf, 4)
    if ver != VERSION or chunk != CHUNK or total != len(buf):
        raise OracleError("bad container header")
    header = buf[CONTAINER_HEADER:CONTAINER_HEADER + HEADER_BYTES]
    off = CONTAINER_HEADER + HEADER_BYTES
    specs = []
    for _ in range(n_fields):
        n_sym, A, _z = struct.unpack_from("<IHH", buf, off)
        f = np.frombuffer(buf, "<u2", A, off + 8).astype(np.int64)
        specs.append((n_sym, A, f))
        off += 8 + 2 * A
    ends = np.frombuffer(buf, "<u4", n_chunks, off).astype(np.int64)
    k = 0
    fields = []
    for n_sym, A, f in specs:
        lens = [min(CHUNK, n_sym - i) for i in range(0, n_sym, CHUNK)]
        pays = []
        for _ in lens:
            a = int(ends[k - 1]) if k else 0
            pays.append(np.frombuffer(buf, "<u2", (int(ends[k]) - a) // 2, pay_off + a))
            k += 1
        syms = rans_decode(pays, lens, f)
        fields.append((np.concatenate(syms) if syms else np.zeros(0, np.uint8), A))
    if k != n_chunks:
        raise OracleError("chunk count mismatch")
    out = merge_fields(header, fields, params, slot, T)
    if len(out) != stream_bytes:
        raise OracleError("stream length mismatch")
    return out


def container_bound(params, slot, T: int) -> int:
    """Largest container a stream of this shape can need: one word per symbol
    plus every chunk's 64 states."""
    s1, w1, tc = split_rows(T, params.sink, params.window)
    n_pt = (s1 + w1) * params.F
    sizes = [n_pt] * params.elem_bytes + [tc * slot.n_act] * 8 + [tc * slot.G] * slot.n_act
    alph = [256] * (params.elem_bytes + 8) + [1 << int(slot.widths[g]) for g in slot.active_groups]
    n_chunks = sum((n + CHUNK - 1) // CHUNK for n in sizes)
    head = CONTAINER_HEADER + HEADER_BYTES + sum(8 + 2 * a for a in alph) + 4 * n_chunks
    return (head + 15) // 16 * 16 + sum(2 * n for n in sizes) + 4 * LANES * n_chunks + 15
