"""Shared helpers of the GPU parity tests (device setup, error measures)."""
import sys

import numpy as np
import torch

import synth


def rel_frob(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.linalg.norm(want)
    return float(np.linalg.norm(got - want) / (den if den > 0 else 1.0))


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def x_tensor(raw, dtype, device):
    """Device tensor from synth.make_x's raw array (float32 / float16 / bf16 bits)."""
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(raw)).to(device)
    if dtype == "f16":
        return torch.from_numpy(np.ascontiguousarray(raw)).to(device)
    t = torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).to(device)
    return t.view(torch.bfloat16)


TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def same_products(y_index, y_slot, prefill):
    """Slot codes name the same codewords as codebook indices, so both formats form
    the same exact products.  The decode paths and the row-order prefill kernel run
    the same kernel on both: bit-equal outputs.  The prefill of a slot-code layer
    runs the shared-tile kernel (another fp32 summation order): within 1e-5."""
    if not prefill:
        return bool(torch.equal(y_index, y_slot))
    return rel_frob(to_f64(y_slot), to_f64(y_index)) <= 1e-5


def to_f64(t):
    return t.detach().to(torch.float64).cpu().numpy()


def fp32_to_f16_rn(y32):
    return np.asarray(y32, dtype=np.float32).astype(np.float16).astype(np.float64)


def fp32_to_bf16_rn(y32):
    from oracle import glq as og
    return og.bf16_bits_to_f64(og.fp32_to_bf16_bits(np.asarray(y32, dtype=np.float32)))


def layer_from(workload_key, k):
    w = synth.WORKLOADS[workload_key]
    return synth.make_layer(w.layers[k], w.resid_bits, w.seed, k)
