"""Helpers for the GPU parity tests: oracle artifacts, device buffers, and
running the library's entry points on cuda:0 (torch only allocates memory and
provides the stream)."""
from __future__ import annotations

import functools

import numpy as np
import torch

import kv_cache_transform_amd as K
import oracle.kvtc_oracle as O
import synth

DEV = "cuda:0"


def oracle_params(w, max_bits=8) -> O.Params:
    dt = O.DTYPE_F32 if w.dtype == "f32" else O.DTYPE_BF16
    return O.Params(w.n_layers, w.kv_heads, w.head_dim, w.sink, w.window, w.group, max_bits,
                    w.bits_per_value, dt)


@functools.lru_cache(maxsize=None)
def oracle_slot(wname: str, layer: int, kind: int, calib_tokens: int) -> O.Slot:
    w = synth.workload(wname)
    x = synth.gen_kv(w, layer, kind, synth.ROLE_CALIB, calib_tokens)
    return O.calibrate(x, oracle_params(w), layer, kind)


def oracle_artifact(wname: str, slots, calib_tokens=None) -> O.Artifact:
    w = synth.workload(wname)
    n = calib_tokens or w.calib_tokens
    return O.Artifact(oracle_params(w), {(l, k): oracle_slot(wname, l, k, n) for l, k in slots})


@functools.lru_cache(maxsize=None)
def oracle_artifact_set(wname: str, slots: tuple, calib_tokens: int, shared: bool,
                        global_budget: bool) -> O.Artifact:
    """An artifact from the oracle's calibration of a tensor set (shared basis
    per kind and/or one bit budget over the set, at most 256 components per
    tensor)."""
    w = synth.workload(wname)
    ins = [(l, k, synth.gen_kv(w, l, k, synth.ROLE_CALIB, calib_tokens)) for l, k in slots]
    op = oracle_params(w)
    return O.Artifact(op, O.calibrate_set(ins, op, shared_basis=shared, global_budget=global_budget,
                                          max_active=256 // w.group))


def to_dev_bytes(b: bytes, pad: int = 0) -> torch.Tensor:
    t = torch.zeros(len(b) + pad, dtype=torch.uint8)
    t[: len(b)] = torch.frombuffer(bytearray(b), dtype=torch.uint8)
    return t.to(DEV)


def storage_to_dev(store: np.ndarray) -> torch.Tensor:
    if store.dtype == np.uint16:
        return torch.from_numpy(store.view(np.int16).copy()).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(store, np.float32)).to(DEV)


class DevCodec:
    """A library codec loaded from artifact bytes and uploaded to cuda:0."""

    def __init__(self, art_bytes: bytes):
        self.codec = K.Codec.load(art_bytes)
        n = self.codec.state_bytes()
        self.state = torch.empty(n, dtype=torch.uint8, device=DEV)
        self.codec.upload(self.state, n, torch.cuda.current_stream())
        self.ws = torch.zeros(K.kvtc_workspace_bytes(K.KVTC_MAX_JOBS) // 4, dtype=torch.int32,
                              device=DEV)

    def status(self, n):
        return K.kvtc_read_device_status(self.ws, n, torch.cuda.current_stream())

    def encode(self, items):
        """items: list of (layer, kind, dev_tensor [T, F]). Returns stream bytes list."""
        jobs, bufs = [], []
        for layer, kind, x in items:
            n = self.codec.encoded_bytes(layer, kind, x.shape[0])
            buf = torch.full((max(n, 16),), 0xEE, dtype=torch.uint8, device=DEV)
            bufs.append((buf, n))
            jobs.append(K.make_job(layer, kind, x.shape[0], x, buf, n))
        self.codec.encode(jobs, self.ws, torch.cuda.current_stream())
        st = self.status(len(jobs))
        assert np.all(st == 0), st
        return [bytes(b[:n].cpu().numpy().tobytes()) for b, n in bufs]

    def out_buffer(self, T, F, out_dtype, rows=None):
        rows = T if rows is None else rows
        dt = torch.float32 if out_dtype == K.KVTC_F32 else torch.int16
        return torch.full((max(rows, 1), F), -7, dtype=dt, device=DEV) if dt == torch.int16 else \
            torch.full((max(rows, 1), F), -7.0, dtype=dt, device=DEV)

    def decode(self, items, out_dtype, F, paging=None, two_stage=False, stg_fill=0, schedule="fused"):
        """items: list of (layer, kind, T, stream bytes). paging: list of
        (block_table dev tensor, block_size, n_blocks) per item or None.
        two_stage: the explicit kvtc_decode_unpack / kvtc_decode_restore calls,
        else kvtc_decode with the workspace of `schedule` (see decode_jobs).
        stg_fill: byte the staging memory holds before the call (0xFF makes
        every float read from it that stage 1 did not write a NaN).
        Returns (outputs, status)."""
        jobs, outs, keep = [], [], []
        for i, (layer, kind, T, sb) in enumerate(items):
            src = to_dev_bytes(sb, 16)
            keep.append(src)
            if paging and paging[i] is not None:
                bt, bs, nblk = paging[i]
                out = self.out_buffer(T, F, out_dtype, rows=nblk * bs)
                jobs.append(K.make_job(layer, kind, T, src, out, out.numel() * out.element_size(),
                                       bt, bs, nblk))
            else:
                out = self.out_buffer(T, F, out_dtype)
                jobs.append(K.make_job(layer, kind, T, src, out, out.numel() * out.element_size()))
            outs.append(out)
        s = torch.cuda.current_stream()
        if two_stage:
            n = self.codec.staging_bytes(jobs)
            stg = torch.full((max(n, 256),), stg_fill, dtype=torch.uint8, device=DEV)
            self.codec.decode_unpack(jobs, out_dtype, stg, stg.numel(), self.ws, s)
            self.codec.decode_restore(jobs, out_dtype, stg, stg.numel(), self.ws, s)
            st = self.status(len(jobs))
        else:
            st = self.decode_jobs(jobs, out_dtype, stg_fill, schedule)
        torch.cuda.synchronize()
        return outs, st

    def decode_jobs(self, jobs, out_dtype, stg_fill=0, schedule="fused"):
        """kvtc_decode of prepared jobs with a workspace of its own (status words
        zeroed, any staging part filled with stg_fill): schedule "fused" gives it
        kvtc_workspace_bytes(n) (the single-launch schedule), "staged"
        kvtc_decode_workspace_bytes (the two-stage schedule). Returns the status."""
        s = torch.cuda.current_stream()
        full = self.codec.decode_workspace_bytes(jobs)
        assert full > 0
        n = K.kvtc_workspace_bytes(len(jobs)) if schedule == "fused" else full
        dws = torch.zeros((n + 3) // 4, dtype=torch.int32, device=DEV)
        dws.view(torch.uint8)[K.kvtc_workspace_bytes(len(jobs)):].fill_(stg_fill)
        self.codec.decode(jobs, out_dtype, dws, n, s)
        return K.kvtc_read_device_status(dws, len(jobs), s)


def bf16_out_to_f64(t: torch.Tensor) -> np.ndarray:
    return O.bf16_to_f32(t.cpu().numpy().view(np.uint16)).astype(np.float64)


def code_stats(gpu_stream: bytes, ref: O.EncodeResult, params: O.Params, slot: O.Slot, T: int):
    codes, shift, scale = O.read_records(gpu_stream, params, slot, T)
    d = codes.astype(np.int64) - ref.codes.astype(np.int64)
    return int(np.count_nonzero(d)), int(d.size), int(np.abs(d).max(initial=0)), shift, scale
