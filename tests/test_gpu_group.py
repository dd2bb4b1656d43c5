"""GPU parity of glq_e8rht_linear_group: several E8RHTLinear forwards in one pair of
launches at B = 1, checked layer by layer against the fp64 oracle.

glq 0.5.1, "How it works" and "Inference kernels" (each y_k = RHT_out(RHT_in(x_k)
W~_k^T)); "Advanced -> CUDA-graph decode wrapper" (a B = 1 decode step of a small
model is bound by its launches, which the group shares).  Tolerance: relative
Frobenius error of fp32 y_k <= 1e-3 (the decode bound); fp16 / bf16 outputs equal
the nearest-even rounding of the library's own fp32 output.  Where the group keeps
every layer's own launch plan (its grids fit the device together) each y_k is also
bit-equal to glq_e8rht_linear's; with shared CUs the row blocks differ and only the
fp32 summation order of the output transform changes.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import glq as og
from gpu_util import fp32_to_bf16_rn, fp32_to_f16_rn, layer_from, rel_frob, say, to_f64, x_tensor

pytestmark = pytest.mark.gpu
glq = pytest.importorskip("e8_lattice_codebook_amd")

DECODE_TOL = 1e-3
BLOCK = synth.WORKLOADS["smollm3_block"]
HOST = {}


def host_layer(key, k):
    if (key, k) not in HOST:
        HOST[(key, k)] = layer_from(key, k)
    return HOST[(key, k)]


def oracle_y(layer, x64):
    return og.linear(x64, layer.sign_in, layer.sign_out, layer.n_pad, layer.m, layer.idx0, layer.idx1,
                     layer.resid_bits, layer.wscale, layer.resid_scale)


def check_group(cb, key, ks, B=1, x_of=None, slot=True, own_plans=None):
    """Run layers ks of workload key as one group; every output against the oracle and
    against the single-layer call.  x_of[k]: which layer's activations layer k reads
    (the same tensor for linears that share their input)."""
    w = synth.WORKLOADS[key]
    hosts = [host_layer(key, k) for k in ks]
    qls = [glq.QuantizedLayer.from_synth(h, cb) for h in hosts]
    if slot:
        qls = [q.to_slot_codes() for q in qls]
    src = {k: (x_of or {}).get(k, k) for k in ks}
    xs64, xdev = {}, {}
    for k in set(src.values()):
        n = host_layer(key, k).n
        x64, raw = synth.make_x(n, B, w.act_dtype, w.seed, k)
        xs64[k] = x64
        xdev[k] = x_tensor(raw, w.act_dtype, "cuda:0")
    xs = [xdev[src[k]] for k in ks]
    say("group", key, ks, "B", B, "slot" if slot else "index")
    ys = glq.e8rht_linear_group(qls, xs, torch.float32)
    singles = [glq.e8rht_linear(q, x, torch.float32) for q, x in zip(qls, xs)]
    torch.cuda.synchronize()
    for j, k in enumerate(ks):
        want = oracle_y(hosts[j], xs64[src[k]])
        err = rel_frob(to_f64(ys[j]), want)
        say("  layer", k, "rel_frob", err)
        assert err <= DECODE_TOL, (key, k, err)
        if own_plans:
            assert torch.equal(ys[j], singles[j]), (key, k)
        else:
            assert rel_frob(to_f64(ys[j]), to_f64(singles[j])) <= 1e-6, (key, k)
    # 16-bit outputs: one nearest-even rounding of the group's own fp32 result
    for dt, rn in ((torch.float16, fp32_to_f16_rn), (torch.bfloat16, fp32_to_bf16_rn)):
        y16 = glq.e8rht_linear_group(qls, xs, dt)
        torch.cuda.synchronize()
        for j in range(len(ks)):
            assert np.array_equal(to_f64(y16[j]), rn(to_f64(ys[j]))), (key, ks[j], dt)
    return ys


def test_qkv_shared_input(gpu_codebooks):
    # q, k and v read the same activations; their grids (64 + 16 + 16 workgroups) fit
    # the device together, so each keeps its own plan
    check_group(gpu_codebooks, "smollm3_block", [0, 1, 2], x_of={1: 0, 2: 0}, own_plans=True)


def test_gate_up_shared_input_shared_cus(gpu_codebooks):
    # gate and up each want every CU: the group splits the CUs between them
    check_group(gpu_codebooks, "smollm3_block", [4, 5], x_of={5: 4})


def test_uneven_cu_shares(gpu_codebooks):
    # gate, up and k: shares of 126, 126 and 3 CUs, row counts that are no power of two
    check_group(gpu_codebooks, "smollm3_block", [4, 5, 1], x_of={5: 4, 1: 4})


def test_devstral_gate_up_shared_cus(gpu_codebooks):
    # two 32768 x 8192 layers (64 lanes per row, bf16): 128 CUs each, 256 row-steps per
    # workgroup, so the waves take their rows in chunks from the LDS counter
    check_group(gpu_codebooks, "devstral_mlp", [0, 1], x_of={1: 0})


def test_four_layers_own_inputs_codebook_indices(gpu_codebooks):
    check_group(gpu_codebooks, "smollm3_block", [0, 1, 2, 3], slot=False, own_plans=True)


def test_single_layer_group(gpu_codebooks):
    check_group(gpu_codebooks, "smollm3_block", [6], own_plans=True)


def test_other_recipes(gpu_codebooks):
    # 16-bit residual (4 bpw, fp16) and no residual (2 bpw, fp32)
    check_group(gpu_codebooks, "smollm2_up", [0], own_plans=True)
    check_group(gpu_codebooks, "tiny", [0], slot=False, own_plans=True)


def test_fallback_batch_and_mixed_n_pad(gpu_codebooks):
    # B = 3 on layers the int8 path does not take (q, k, v: the staged decode) and layers
    # of different n_pad run one call after another: the single calls' bits
    check_group(gpu_codebooks, "smollm3_block", [0, 1, 2], B=3, x_of={1: 0, 2: 0}, own_plans=True)
    check_group(gpu_codebooks, "smollm3_block", [3, 6], own_plans=True)


def test_int8_group_own_plans(gpu_codebooks):
    # 2 <= B <= 16 with every layer on the int8 path: one GEMV launch for q, k and v at
    # B = 5, whose grids fit the device together (each layer's own plan: single-call bits)
    check_group(gpu_codebooks, "smollm3_block", [0, 1, 2], B=5, x_of={1: 0, 2: 0}, own_plans=True)


@pytest.mark.parametrize("B", [4, 16])
def test_int8_group_devstral_gate_up(gpu_codebooks, B):
    # the Devstral gate and up layers at B = 4 and 16 on shared CUs (128 each)
    check_group(gpu_codebooks, "devstral_mlp", [0, 1], B=B, x_of={1: 0})


def test_int8_group_smollm3_gate_up_uneven(gpu_codebooks):
    # SmolLM3 gate, up and k at B = 5: uneven shares of the CUs
    check_group(gpu_codebooks, "smollm3_block", [4, 5, 1], B=5, x_of={5: 4, 1: 4})


def test_repeat_bit_identical(gpu_codebooks):
    ys1 = check_group(gpu_codebooks, "smollm3_block", [4, 5, 1], x_of={5: 4, 1: 4})
    ys2 = check_group(gpu_codebooks, "smollm3_block", [4, 5, 1], x_of={5: 4, 1: 4})
    assert all(torch.equal(a, b) for a, b in zip(ys1, ys2))


def test_group_errors(gpu_codebooks):
    hosts = [host_layer("smollm3_block", k) for k in (0, 1)]
    qls = [glq.QuantizedLayer.from_synth(h, gpu_codebooks) for h in hosts]
    x = torch.zeros((1, 2048), dtype=torch.float16, device="cuda:0")
    with pytest.raises(glq.GLQError) as e:
        glq.e8rht_linear_group(qls * 3, [x] * 6)
    assert e.value.name == "GLQ_ERR_SHAPE"
    ws = torch.empty(16, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(glq.GLQError) as e:
        glq.e8rht_linear_group(qls, [x, x], workspace=ws)
    assert e.value.name == "GLQ_ERR_WORKSPACE"


def test_unpadded_block_diagonal_layers(gpu_codebooks):
    # unpadded layers (n_pad = n = 5120 = 4096 + 1024, block-diagonal transforms) sharing
    # one input: m = 11008 (8192 + 2048 + 512 + 256) and 2560, 4 bpw, bf16
    hosts = [synth.block_layer(5120, 11008, 16, seed=71), synth.block_layer(5120, 2560, 16, seed=72)]
    qls = [glq.QuantizedLayer.from_synth(h, gpu_codebooks).to_slot_codes() for h in hosts]
    x64, raw = synth.make_x(5120, 1, "bf16", 73, 0)
    x = x_tensor(raw, "bf16", "cuda:0")
    say("group unpadded 5120 -> 11008, 2560")
    ys = glq.e8rht_linear_group(qls, [x, x], torch.float32)
    singles = [glq.e8rht_linear(q, x, torch.float32) for q in qls]
    torch.cuda.synchronize()
    for h, y, y1 in zip(hosts, ys, singles):
        want = og.linear(x64, h.sign_in, h.sign_out, h.n_pad, h.m, h.idx0, h.idx1, h.resid_bits, h.wscale,
                         h.resid_scale, block_diag=True)
        err = rel_frob(to_f64(y), want)
        say("  rel_frob", err)
        assert err <= DECODE_TOL, err
        assert rel_frob(to_f64(y), to_f64(y1)) <= 1e-6


@pytest.mark.parametrize("bpw", [5, 6, 7, 8])
def test_recipes_5_to_8_bpw(gpu_codebooks, bpw):
    # the further 8/16-bit stages of 5-8 bpw in the grouped launch: two layers of one
    # recipe sharing an input, shares of the CUs (16384 + 4096 rows at n_pad 2048)
    hosts = [synth.recipe_layer(2048, 11008, bpw, seed=80 + bpw), synth.recipe_layer(2048, 4096, bpw, seed=90 + bpw)]
    qls = [glq.QuantizedLayer.from_synth(h, gpu_codebooks).to_slot_codes() for h in hosts]
    x64, raw = synth.make_x(2048, 1, "f16", 95, bpw)
    x = x_tensor(raw, "f16", "cuda:0")
    say("group recipes", bpw)
    ys = glq.e8rht_linear_group(qls, [x, x], torch.float32)
    singles = [glq.e8rht_linear(q, x, torch.float32) for q in qls]
    torch.cuda.synchronize()
    for h, y, y1 in zip(hosts, ys, singles):
        want = og.linear(x64, h.sign_in, h.sign_out, h.n_pad, h.m, h.idx0, h.idx1, h.resid_bits, h.wscale,
                         h.resid_scale, extra=h.oracle_extra())
        err = rel_frob(to_f64(y), want)
        say("  rel_frob", err)
        assert err <= DECODE_TOL, (bpw, err)
        assert rel_frob(to_f64(y), to_f64(y1)) <= 1e-6
