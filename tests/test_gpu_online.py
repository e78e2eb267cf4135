"""Online layer-by-layer encode (cuda:0, through the C ABI).

The KV cache is compressed while it is produced (KVTC page, section 2B:
compression fits in the gaps of inference; the KVCodec pages name pipelined
layer-by-layer GPU encoding as the way to keep up with production). Here a
producer writes layer l + 1's K and V (a bf16 GEMM of hidden states by that
layer's projection, standing in for the model) on one stream while layer l
is encoded on another, each encode waiting on its layer's event. The streams
must be byte-identical to one kvtc_encode call over every layer after all of
them are produced, and every status must be OK.
"""
import numpy as np
import pytest
import torch

import kv_cache_transform_amd as K
from gpu_util import DEV, DevCodec, oracle_artifact

pytestmark = pytest.mark.gpu

WL, LAYERS, T, D = "llama31_8b", 4, 2048, 1024


def _produce(h, wk, wv, outs, l):
    torch.matmul(h, wk[l], out=outs[2 * l])
    torch.matmul(h, wv[l], out=outs[2 * l + 1])


def test_online_encode_matches_one_shot():
    art = oracle_artifact(WL, [(l, k) for l in range(LAYERS) for k in (0, 1)], 4096)
    dc = DevCodec(art.serialize())
    F = art.params.F
    g = torch.Generator(device=DEV).manual_seed(7)
    h = torch.randn((T, D), generator=g, device=DEV, dtype=torch.float32).to(torch.bfloat16)
    wk = [(torch.randn((D, F), generator=g, device=DEV) * D ** -0.5).to(torch.bfloat16).contiguous()
          for _ in range(LAYERS)]
    wv = [(torch.randn((D, F), generator=g, device=DEV) * D ** -0.5).to(torch.bfloat16).contiguous()
          for _ in range(LAYERS)]
    kv = torch.empty((2 * LAYERS, T, F), dtype=torch.bfloat16, device=DEV)
    outs = [kv[i] for i in range(2 * LAYERS)]
    sizes = [dc.codec.encoded_bytes(l, k, T) for l in range(LAYERS) for k in (0, 1)]
    offs = np.cumsum([0] + [(n + 255) // 256 * 256 for n in sizes])

    def jobs_for(buf, layers):
        return [[K.make_job(l, k, T, kv[2 * l + k], buf.data_ptr() + int(offs[2 * l + k]), sizes[2 * l + k])
                 for k in (0, 1)] for l in layers]

    # online: producer stream P writes layer l + 1 while stream E encodes layer l
    online = torch.full((int(offs[-1]),), 0xEE, dtype=torch.uint8, device=DEV)
    ws_e = [torch.zeros(K.kvtc_workspace_bytes(2) // 4, dtype=torch.int32, device=DEV)
            for _ in range(LAYERS)]
    sp, se = torch.cuda.Stream(), torch.cuda.Stream()
    ev = [torch.cuda.Event() for _ in range(LAYERS)]
    torch.cuda.synchronize()
    for l, js in enumerate(jobs_for(online, range(LAYERS))):
        with torch.cuda.stream(sp):
            _produce(h, wk, wv, outs, l)
            ev[l].record(sp)
        se.wait_event(ev[l])
        dc.codec.encode(js, ws_e[l], se)       # queued; the host goes on to layer l + 1
    torch.cuda.synchronize()
    st_online = np.concatenate([K.kvtc_read_device_status(w, 2, se) for w in ws_e])
    assert np.all(st_online == 0), st_online

    # one shot: every layer produced, then one encode call
    ref = torch.full_like(online, 0x11)
    kv_online = kv.clone()
    for l in range(LAYERS):
        _produce(h, wk, wv, outs, l)
    all_jobs = [j for js in jobs_for(ref, range(LAYERS)) for j in js]
    dc.codec.encode(all_jobs, dc.ws, torch.cuda.current_stream())
    assert np.all(dc.status(len(all_jobs)) == 0)
    torch.cuda.synchronize()
    assert torch.equal(kv, kv_online)          # the producer is deterministic
    for i, n in enumerate(sizes):
        a = online[int(offs[i]):int(offs[i]) + n]
        b = ref[int(offs[i]):int(offs[i]) + n]
        assert torch.equal(a, b), i
