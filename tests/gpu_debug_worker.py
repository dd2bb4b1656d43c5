"""Run by tests/test_gpu_debug.py in a subprocess with GLQ_LIB_VARIANT=debug: the device
bounds checks of the debug build over one call of each path (B = 1 fused decode, B = 5
staged decode, prefill, a grouped B = 1 launch, KV attention with large and small
pages), both index formats where they apply,
each checked against the oracle; prints one line per path and then the violations."""
import os
import sys

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import e8_lattice_codebook_amd as glq  # noqa: E402
import synth  # noqa: E402
from e8_lattice_codebook_amd import _lib  # noqa: E402
from oracle import glq as og  # noqa: E402
from oracle import kv as okv  # noqa: E402

DEV = "cuda:0"


def rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def main():
    lib = _lib.load()
    assert _lib.LIB_PATH.endswith("libglq_mi355x_debug.so"), _lib.LIB_PATH
    assert lib.glq_debug_violations() == 0
    cb = glq.Codebooks(DEV)
    for B, tol in ((1, 1e-3), (5, 1e-3), (40, 5e-3)):
        layer = synth.random_layer(1000, 3000, 8, seed=B, n_pad=1024, m_pad=4096)
        ql = glq.QuantizedLayer.from_synth(layer, cb)
        x64, raw = synth.make_x(1000, B, "f32", B, 8)
        want = og.linear(x64, layer.sign_in, layer.sign_out, layer.n_pad, layer.m, layer.idx0, layer.idx1, 8,
                         layer.wscale, layer.resid_scale)
        for q in (ql, ql.to_slot_codes()):
            y = glq.e8rht_linear(q, torch.from_numpy(raw).to(DEV), torch.float32)
            torch.cuda.synchronize()
            err = rel(y.double().cpu().numpy(), want)
            print("linear B=%d format=%d rel_frob %.3g" % (B, q.index_format, err), flush=True)
            assert err <= tol, (B, err)
    # the grouped B = 1 launches: three layers of one n_pad with uneven CU shares
    hosts = [synth.random_layer(1000, m, 8, seed=60 + k, n_pad=1024, m_pad=mp) for k, (m, mp) in
             enumerate(((3000, 4096), (2500, 4096), (500, 512)))]
    qls = [glq.QuantizedLayer.from_synth(h, cb).to_slot_codes() for h in hosts]
    x64, raw = synth.make_x(1000, 1, "f32", 61, 8)
    x = torch.from_numpy(raw).to(DEV)
    ys = glq.e8rht_linear_group(qls, [x, x, x], torch.float32)
    torch.cuda.synchronize()
    for h, y in zip(hosts, ys):
        want = og.linear(x64, h.sign_in, h.sign_out, h.n_pad, h.m, h.idx0, h.idx1, 8, h.wscale, h.resid_scale)
        err = rel(y.double().cpu().numpy(), want)
        print("group m_pad=%d rel_frob %.3g" % (h.m_pad, err), flush=True)
        assert err <= 1e-3, err
    for page in (16, 4):
        cache = synth.make_kv([300, 41], 2, 128, 2, page, seed=page)
        q64, qraw = synth.make_q(2, 8, 128, "f32", seed=page + 1)
        want = okv.attention_decode(q64, cache.k_idx0, cache.k_idx1, cache.k_scale, cache.v_idx0, cache.v_idx1,
                                    cache.v_scale, cache.resid_scale, cache.block_table, cache.seq_lens,
                                    cache.page_size, 1.0 / np.sqrt(128))
        dc = glq.KVCache.from_synth(cache, cb)
        for c in (dc, dc.to_slot_codes()):
            out = glq.e8kv_attention_decode(c, torch.from_numpy(qraw).to(DEV),
                                            torch.from_numpy(cache.block_table).to(DEV),
                                            torch.from_numpy(cache.seq_lens).to(DEV), 300)
            torch.cuda.synchronize()
            err = rel(out.double().cpu().numpy(), want)
            print("kv page=%d rel_frob %.3g" % (page, err), flush=True)
            assert err <= 1e-3, (page, err)
    v = lib.glq_debug_violations()
    print("violations", v, flush=True)
    assert v == 0, v


if __name__ == "__main__":
    main()
