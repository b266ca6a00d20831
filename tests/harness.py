"""Shared helpers of the GPU parity tests: run one workload step through the
C-ABI binding and through the oracle on the same seeded inputs, and compare.

Only tests import this module. It calls the oracle (CPU) and the product
binding (GPU) side by side; neither of those imports the other.
"""

from __future__ import annotations

import sys
import time

import numpy as np
import torch

import oracle
import paged_kv_cache_165_amd as pa
import workloads as W

ORACLE_DTYPE = {torch.float32: oracle.F32, torch.bfloat16: oracle.BF16, torch.float16: oracle.F16}

# Tolerances on the attention output (float64 oracle as reference):
#   float32 inputs: max-abs error <= 1e-4
#   bfloat16 / float16 inputs with float32 accumulation: max-abs <= 2e-2 and
#   relative RMS ||out - ref|| / ||ref|| <= 1e-2 over the whole output.
TOL_F32_MAX_ABS = 1e-4
TOL_LOW_MAX_ABS = 2e-2
TOL_LOW_REL_RMS = 1e-2


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def host_bits(t: torch.Tensor) -> np.ndarray:
    """Raw storage of a tensor as a numpy array the oracle accepts."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.uint16).numpy()
    return t.numpy()


def raw_equal(a: torch.Tensor, b_host: np.ndarray) -> bool:
    """Bitwise equality of a device tensor with a host array (NaN-safe)."""
    ah = host_bits(a)
    if ah.dtype == np.float32:
        return np.array_equal(ah.view(np.uint32), b_host.view(np.uint32))
    if ah.dtype == np.float16:
        return np.array_equal(ah.view(np.uint16), b_host.view(np.uint16))
    return np.array_equal(ah, b_host)


def compare_attention(out: torch.Tensor, ref: np.ndarray, tag: str = "") -> dict:
    got = out.detach().float().cpu().numpy().astype(np.float64)
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), f"{tag}: non-finite output"
    err = np.abs(got - ref)
    max_abs = float(err.max()) if err.size else 0.0
    den = float(np.linalg.norm(ref))
    rel_rms = float(np.linalg.norm(got - ref) / den) if den > 0 else float(np.linalg.norm(got - ref))
    stats = {"max_abs": max_abs, "rel_rms": rel_rms}
    if out.dtype == torch.float32:
        assert max_abs <= TOL_F32_MAX_ABS, f"{tag}: max-abs {max_abs:.3e} > {TOL_F32_MAX_ABS}"
    else:
        assert max_abs <= TOL_LOW_MAX_ABS, f"{tag}: max-abs {max_abs:.3e} > {TOL_LOW_MAX_ABS}"
        assert rel_rms <= TOL_LOW_REL_RMS, f"{tag}: rel-RMS {rel_rms:.3e} > {TOL_LOW_REL_RMS}"
    return stats


class DeviceCase:
    """One workload's inputs on the GPU plus the host copies the oracle needs."""

    def __init__(self, w: W.Workload, device="cuda", poison=True):
        self.w = w
        v = W.make_values(w, device=device, poison=poison)
        self.q = v["q"]
        self.k_cache = v["k_cache"]
        self.v_cache = v["v_cache"]
        self.write_values = v["writes"]
        self.tables = torch.from_numpy(w.block_tables).to(device)
        self.lens = torch.from_numpy(w.context_lens).to(device)
        self.pairs = torch.from_numpy(w.cow_pairs.astype(np.int32)).to(device)
        self.slots = [torch.from_numpy(op.slots.astype(np.int32)).to(device) for op in w.writes]
        self.out = torch.empty_like(self.q)
        self.workspace = pa.alloc_workspace(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim,
                                            w.max_context_len, w.block_size, w.partition_size, self.q.dtype,
                                            device=device)

    def gpu_step(self, partition_size=None, decode=True):
        w = self.w
        if len(w.cow_pairs):
            pa.copy_blocks(self.k_cache, self.v_cache, self.pairs)
        for slots, (k, v) in zip(self.slots, self.write_values):
            pa.write_cache(k, v, self.k_cache, self.v_cache, slots)
        if decode:
            part = w.partition_size if partition_size is None else partition_size
            ws = self.workspace
            need = pa.workspace_size(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim, w.max_context_len,
                                     w.block_size, part, self.q.dtype)
            if need > ws.numel():
                ws = torch.empty(need, dtype=torch.uint8, device=self.q.device)
            pa.decode(self.out, self.q, self.k_cache, self.v_cache, self.tables, self.lens, w.scale,
                      max_context_len=w.max_context_len, partition_size=part, workspace=ws)
        return self.out


def oracle_step(w: W.Workload, q_h, kc_h, vc_h, write_values_h):
    """The same step on the CPU: copy, writes, then float64 decode."""
    dt = {"f32": oracle.F32, "bf16": oracle.BF16}[w.dtype]
    kc, vc = oracle.copy_blocks(kc_h, vc_h, w.cow_pairs)
    for op, (k, v) in zip(w.writes, write_values_h):
        kc, vc = oracle.write_cache(k, v, kc, vc, op.slots, w.block_size)
    t0 = time.perf_counter()
    ref = oracle.paged_decode(q_h, kc, vc, w.block_tables, w.context_lens, w.scale, w.block_size, dt)
    return kc, vc, ref, time.perf_counter() - t0
