"""Helpers for the GPU parity tests: move seeded inputs to the device and
bring results back.  Tests compare the HIP path (through the C ABI) with the
oracle on the same seeded inputs; nothing here computes expected values."""
import sys

import numpy as np
import torch

from fp4_quantized_moe_amd import _lib as Q


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_act(a):
    """synthetic.Activation -> device tensor in its storage dtype."""
    if a.bits is not None:
        return torch.from_numpy(a.bits.view(np.int16).copy()).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a.f32)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def nvfp4_host(q):
    return host(q.codes), host(q.scales), host(q.gscale)


def rel_err(y, y_ref):
    y_ref = np.asarray(y_ref, dtype=np.float64)
    return float(np.max(np.abs(np.asarray(y, np.float64) - y_ref)) / max(np.max(np.abs(y_ref)), 1e-300))


def quantize_weights_gpu(w_dev, n_seg):
    """[E, N, K] device weights -> (codes [E,N,K/2], scales [E,N,K/16], gscale [E*n_seg])
    with one tensor scale per (expert, segment)."""
    E, N, K = w_dev.shape
    q, _ = Q.quantize_nvfp4(w_dev.reshape(E * n_seg, N // n_seg, K))
    return q.codes.reshape(E, N, K // 2), q.scales.reshape(E, N, K // 16), q.gscale
