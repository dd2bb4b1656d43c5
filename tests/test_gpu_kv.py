"""GPU parity of decode attention over an E8-compressed paged K/V cache against the
fp64 oracle (Glq v0.5.0 release notes, "Highlights"; glq 0.5.1, "KV cache
compression": the cache dequantized inside the attention kernel, the 8-point
inverse Hadamard, flash-decoding over chunks of the context).

Tolerance: the query is rotated once and held in fp16 (products with the exact
fp16 codeword values accumulate in fp32), scores and sums are fp32 and
exp is the hardware's; the output's relative Frobenius error is bounded by 1e-3,
the decode bound of the linear.  Slot-code caches give bit for bit the output of
codebook-index caches, and repeated calls are bit-identical.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import kv as okv
from gpu_util import TORCH_DT, rel_frob, say, to_f64

pytestmark = pytest.mark.gpu
glq = pytest.importorskip("e8_lattice_codebook_amd")
DEV = "cuda:0"


def _oracle(cache, q64, sm_scale):
    return okv.attention_decode(q64, cache.k_idx0, cache.k_idx1, cache.k_scale, cache.v_idx0, cache.v_idx1,
                                cache.v_scale, cache.resid_scale, cache.block_table, cache.seq_lens,
                                cache.page_size, sm_scale)


def _run(gpu_codebooks, cache, q_raw, qdt, max_len=None, out_dtype=torch.float32, slot=False):
    dc = glq.KVCache.from_synth(cache, gpu_codebooks)
    if slot:
        dc = dc.to_slot_codes()
    q = torch.from_numpy(np.ascontiguousarray(q_raw).view(np.int16) if qdt == "bf16" else q_raw).to(DEV)
    if qdt == "bf16":
        q = q.view(torch.bfloat16)
    bt = torch.from_numpy(cache.block_table).to(DEV)
    lens = torch.from_numpy(cache.seq_lens).to(DEV)
    ml = int(cache.seq_lens.max()) if max_len is None else max_len
    out = glq.e8kv_attention_decode(dc, q, bt, lens, ml, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out


CASES = [  # (seq_lens, Hkv, G, D, stages, page_size, q dtype)
    ([1], 1, 1, 128, 2, 16, "f32"),
    ([17, 300], 2, 4, 128, 2, 16, "bf16"),
    ([1000, 5, 257], 4, 4, 128, 2, 16, "bf16"),
    ([5000], 4, 4, 128, 1, 64, "bf16"),
    ([700, 64], 2, 2, 64, 2, 16, "f16"),
    ([333], 1, 8, 128, 2, 1, "bf16"),
    ([129, 2048], 2, 8, 64, 1, 32, "f32"),
    ([4096, 1, 77, 640], 8, 1, 128, 2, 16, "bf16"),
]


@pytest.mark.parametrize("lens,Hkv,G,D,stages,P,qdt", CASES)
def test_attention_matches_oracle(gpu_codebooks, lens, Hkv, G, D, stages, P, qdt):
    say("kv attention", lens, Hkv, G, D, stages, P, qdt)
    cache = synth.make_kv(lens, Hkv, D, stages, P, seed=sum(lens) + G)
    q64, raw = synth.make_q(len(lens), Hkv * G, D, qdt, seed=D + G)
    out = _run(gpu_codebooks, cache, raw, qdt)
    outs = _run(gpu_codebooks, cache, raw, qdt, slot=True)
    assert torch.equal(out, outs)
    want = _oracle(cache, q64, 1.0 / np.sqrt(D))
    err = rel_frob(to_f64(out), want)
    say("  rel_frob", err)
    assert err <= 1e-3, err


@pytest.mark.parametrize("resid_scale", [1.0, 0.5, 0.125, 0.0625, 0.3])
def test_resid_scales(gpu_codebooks, resid_scale):
    # two stages with other residual scales: powers of two 2^-k (k <= 4) merge the
    # stages' integer codes exactly, any other scale combines them in fp16 (0.3 is
    # rounded to fp16 once); both formats, within the same 1e-3 of the oracle
    say("kv resid_scale", resid_scale)
    cache = synth.make_kv([700, 33], 2, 128, 2, 16, seed=61)
    cache.resid_scale = resid_scale
    q64, raw = synth.make_q(2, 8, 128, "bf16", seed=62)
    out = _run(gpu_codebooks, cache, raw, "bf16")
    outs = _run(gpu_codebooks, cache, raw, "bf16", slot=True)
    assert torch.equal(out, outs)
    err = rel_frob(to_f64(out), _oracle(cache, q64, 1.0 / np.sqrt(128)))
    say("  rel_frob", err)
    assert err <= 1e-3, err


@pytest.mark.parametrize("D,G", [(64, 2), (128, 4)])
def test_more_units_than_compute_units(gpu_codebooks, D, G):
    # 40 sequences x 8 KV heads: more (sequence, head, chunk) units than compute units,
    # so workgroups take several units in turn (the waves' results merged in turns on
    # all but the last, the image reloaded after the last one's merge); ragged lengths
    # include 1-token and page-boundary sequences
    lens = [1, 16, 17, 300, 255, 33] + list(np.random.default_rng(D).integers(1, 400, size=34))
    say("kv many units", D, G, len(lens))
    cache = synth.make_kv(lens, 8, D, 2, 16, seed=71 + D)
    q64, raw = synth.make_q(len(lens), 8 * G, D, "bf16", seed=72)
    out = _run(gpu_codebooks, cache, raw, "bf16")
    outs = _run(gpu_codebooks, cache, raw, "bf16", slot=True)
    assert torch.equal(out, outs)
    err = rel_frob(to_f64(out), _oracle(cache, q64, 1.0 / np.sqrt(D)))
    say("  rel_frob", err)
    assert err <= 1e-3, err


def test_smollm3_shape_16k(gpu_codebooks):
    # the timed shape: SmolLM3-3B attention, 16 query heads on 4 KV heads, head_dim
    # 128, 4 sequences of 16k tokens, 4 bpw cache, bf16 query (the first layer's cache
    # and query of the benchmark).  fp32 output within 1e-3 of the oracle; the bf16
    # output is its nearest-even rounding; slot codes (what is timed) give the same
    # bits as codebook indices
    cache = synth.make_kv([16384] * 4, 4, 128, 2, 16, seed=2000, spare_pages=0)
    q64, raw = synth.make_q(4, 16, 128, "bf16", seed=2999)
    out = _run(gpu_codebooks, cache, raw, "bf16")
    outs = _run(gpu_codebooks, cache, raw, "bf16", slot=True)
    assert torch.equal(out, outs)
    want = _oracle(cache, q64, 1.0 / np.sqrt(128))
    err = rel_frob(to_f64(out), want)
    say("  rel_frob", err)
    assert err <= 1e-3, err
    ob = _run(gpu_codebooks, cache, raw, "bf16", out_dtype=torch.bfloat16, slot=True)
    assert torch.equal(ob.view(torch.int16), out.to(torch.bfloat16).view(torch.int16))


def test_repeat_is_bit_identical_and_out_dtypes(gpu_codebooks):
    cache = synth.make_kv([3000, 40], 2, 128, 2, 16, seed=41)
    q64, raw = synth.make_q(2, 8, 128, "bf16", seed=42)
    a = _run(gpu_codebooks, cache, raw, "bf16")
    b = _run(gpu_codebooks, cache, raw, "bf16")
    assert torch.equal(a, b)
    for dt in ("f16", "bf16"):
        o = _run(gpu_codebooks, cache, raw, "bf16", out_dtype=TORCH_DT[dt])
        r = a.to(TORCH_DT[dt])  # one nearest-even rounding of the fp32 result
        assert torch.equal(o.view(torch.int16), r.view(torch.int16))


def test_empty_and_clamped_sequences(gpu_codebooks):
    cache = synth.make_kv([50, 20], 1, 64, 2, 16, seed=51)
    q64, raw = synth.make_q(2, 2, 64, "f32", seed=52)
    lens = cache.seq_lens.copy()
    cache.seq_lens[:] = [0, 20]
    out = _run(gpu_codebooks, cache, raw, "f32", max_len=50)
    assert torch.count_nonzero(out[0]) == 0
    want = _oracle(synth.KVCache(1, 64, 16, 2, cache.k_idx0, cache.k_idx1, cache.v_idx0, cache.v_idx1, cache.k_scale,
                                 cache.v_scale, cache.block_table[1:], cache.seq_lens[1:]), q64[1:], 0.125)
    assert rel_frob(to_f64(out[1:]), want) <= 1e-3
    # seq_lens above max_seq_len are clamped to it
    cache.seq_lens[:] = lens
    out = _run(gpu_codebooks, cache, raw, "f32", max_len=30)
    cache.seq_lens[:] = [30, 20]
    want = _oracle(cache, q64, 0.125)
    assert rel_frob(to_f64(out), want) <= 1e-3
