"""Helpers for the GPU parity tests: move generator arrays to the device, run
the HIP path through the C-ABI binding, compare with the oracle."""

from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads as W

ATOL_F32 = 2e-3          # max-abs bound on the attention output (FP32 out)
RTOL_REPORT = 1e-2       # relative bound, denominator max(|ref|, 1e-2)
BF16_REL = 2.0 ** -8     # extra relative room for BF16 output rounding


def dev16(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).to(device)


def dev32(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def host16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


class DeviceBatch:
    """A DecodeBatch uploaded to the GPU."""

    def __init__(self, batch: W.DecodeBatch, device="cuda"):
        self.h = batch
        self.q = dev16(batch.q, device)
        self.k_pool = dev16(batch.k_pool, device)
        self.v_pool = dev16(batch.v_pool, device)
        self.bt = dev32(batch.block_tables, device)
        self.lens = dev32(batch.seq_lens, device)
        self.k_new = dev16(batch.k_new, device) if batch.k_new is not None else None
        self.v_new = dev16(batch.v_new, device) if batch.v_new is not None else None


def gpu_decode(db: DeviceBatch, pages_per_split=0, out_dtype=torch.float32, max_seq_len=None):
    from paged_kv_decode_07_amd import binding as pa
    msl = db.h.max_seq_len if max_seq_len is None else max_seq_len
    out = pa.decode_attention(db.q, db.k_pool, db.v_pool, db.bt, db.lens, msl,
                              scale=db.h.scale, out_dtype=out_dtype,
                              pages_per_split=pages_per_split)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def gpu_append(db: DeviceBatch):
    from paged_kv_decode_07_amd import binding as pa
    pa.append_kv(db.k_new, db.v_new, db.k_pool, db.v_pool, db.bt, db.lens)
    torch.cuda.synchronize()


def oracle_decode(batch: W.DecodeBatch, sequences=None, k_pool=None, v_pool=None):
    return oracle.decode_attention(batch.q, batch.k_pool if k_pool is None else k_pool,
                                   batch.v_pool if v_pool is None else v_pool,
                                   batch.block_tables, batch.seq_lens, batch.scale,
                                   sequences=sequences)


def assert_close(got: np.ndarray, ref: np.ndarray, bf16_out=False, where=""):
    """Max-abs 2e-3 (plus BF16 output rounding when the output is BF16)."""
    assert np.all(np.isfinite(got)), f"non-finite output {where}"
    err = np.abs(got - ref)
    tol = ATOL_F32 + (BF16_REL * np.abs(ref) if bf16_out else 0.0)
    worst = np.unravel_index(np.argmax(err - tol), err.shape)
    assert np.all(err <= tol), (
        f"{where}: max-abs {err.max():.3e} at {worst} (got {got[worst]}, ref {ref[worst]})")
    rel = err / np.maximum(np.abs(ref), 1e-2)
    if not bf16_out:
        assert rel.max() <= RTOL_REPORT, f"{where}: max-rel {rel.max():.3e}"
    return float(err.max()), float(rel.max())


def gpu_fused(db: DeviceBatch, pages_per_split=0, out_dtype=torch.float32):
    """Fused append + decode in one call; pools of ``db`` are updated in place."""
    from paged_kv_decode_07_amd import binding as pa
    out = pa.append_decode_attention(db.q, db.k_new, db.v_new, db.k_pool, db.v_pool, db.bt,
                                     db.lens, db.h.max_seq_len, scale=db.h.scale,
                                     out_dtype=out_dtype, pages_per_split=pages_per_split)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)
