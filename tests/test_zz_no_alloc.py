"""kvtc_decode_noalloc, the decode entry point that allocates nothing (its
status words and sink live in a static device array), against kvtc_decode
with a caller's workspace (the same fused schedule) on cuda:0, through the
C ABI: two calls in a row, the second with fewer jobs and tokens, f32 output
and one stream with a corrupted header; outputs bit for bit, statuses equal."""
import numpy as np
import pytest
import torch

import kv_cache_transform_amd as K
import oracle.kvtc_oracle as O
import synth
from gpu_util import DEV, DevCodec, oracle_artifact, to_dev_bytes

pytestmark = pytest.mark.gpu

WL, SLOTS = "odd3_bf16", [(0, 0), (0, 1)]


def _streams(w, art, T, reqs):
    out = []
    for (l, k) in SLOTS:
        for r in range(reqs):
            store = synth.storage(w, synth.gen_kv(w, l, k, synth.ROLE_EVAL, T, r))
            out.append((l, k, O.encode(store, art.params, art.slots[(l, k)], l, k).stream))
    return out


def _jobs(items, T, F, out_dtype, keep):
    dt = torch.float32 if out_dtype == K.KVTC_F32 else torch.int16
    jobs, outs = [], []
    for l, k, sb in items:
        src = to_dev_bytes(sb, 16)
        out = torch.full((T, F), -7, dtype=dt, device=DEV)
        keep.append(src)
        outs.append(out)
        jobs.append(K.make_job(l, k, T, src, out, out.numel() * out.element_size()))
    return jobs, outs


def test_noalloc_decode_matches_decode():
    w = synth.workload(WL)
    art = oracle_artifact(WL, SLOTS)
    dc = DevCodec(art.serialize())
    F = art.params.F
    s = torch.cuda.current_stream()
    calls = [(1100, 2, K.KVTC_BF16, False), (700, 1, K.KVTC_F32, True)]
    for T, reqs, od, corrupt in calls:
        print(f"noalloc call: T={T} jobs={len(SLOTS) * reqs} out={od} corrupt={corrupt}", flush=True)
        items = _streams(w, art, T, reqs)
        if corrupt:   # the magic of the first stream's header
            l, k, sb = items[0]
            items[0] = (l, k, b"\x00" + sb[1:])
        keep = []
        jobs_a, outs_a = _jobs(items, T, F, od, keep)
        jobs_b, outs_b = _jobs(items, T, F, od, keep)
        n = len(jobs_a)
        nws = K.kvtc_workspace_bytes(n)
        dws = torch.zeros((nws + 3) // 4, dtype=torch.int32, device=DEV)
        dc.codec.decode(jobs_a, od, dws, nws, s)
        st_a = K.kvtc_read_device_status(dws, n, s)
        d_status = torch.full((n,), 12345, dtype=torch.int32, device=DEV)
        dc.codec.decode_noalloc(jobs_b, od, d_status, s)
        torch.cuda.synchronize()
        st_b = d_status.cpu().numpy()
        assert np.array_equal(st_a, st_b), (st_a, st_b)
        assert (st_b[0] == K.KVTC_E_CORRUPT) if corrupt else np.all(st_b == 0), st_b
        assert np.all(st_b[1:] == 0), st_b
        for a, b in zip(outs_a, outs_b):
            assert torch.equal(a, b)
    # without a status output the call still decodes
    jobs_c, outs_c = _jobs(_streams(w, art, 300, 1), 300, F, K.KVTC_BF16, [])
    dc.codec.decode_noalloc(jobs_c, K.KVTC_BF16, None, s)
    torch.cuda.synchronize()
    assert all(bool((o != -7).any()) for o in outs_c)


def test_noalloc_decode_rejects_more_jobs_than_its_array_holds():
    w = synth.workload(WL)
    art = oracle_artifact(WL, SLOTS)
    dc = DevCodec(art.serialize())
    (l, k, sb), = _streams(w, art, 64, 1)[:1]
    src = to_dev_bytes(sb, 16)
    out = torch.zeros((64, art.params.F), dtype=torch.int16, device=DEV)
    job = K.make_job(l, k, 64, src, out, out.numel() * 2)
    with pytest.raises(K.KvtcError) as e:
        dc.codec.decode_noalloc([job] * (K.KVTC_MAX_JOBS + 1), K.KVTC_BF16, None, torch.cuda.current_stream())
    assert e.value.status == K.KVTC_E_CAPACITY
