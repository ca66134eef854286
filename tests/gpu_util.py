"""Helpers shared by the GPU parity tests (comparison metrics and transfers)."""
import numpy as np

# Relative Frobenius tolerances: fp64 values must agree with the fp64 oracle
# to 1e-12; fp32 values (oracle fed the same fp32-rounded inputs) to 2e-5.
TOL = {"f64": 1e-12, "f32": 2e-5}


def rel(a, b):
    a = np.asarray(a, dtype=np.float64).reshape(-1)
    b = np.asarray(b, dtype=np.float64).reshape(-1)
    nb = np.linalg.norm(b)
    d = np.linalg.norm(a - b)
    return d / nb if nb > 0 else d


def dev(a, dtype):
    import torch
    t = torch.float64 if dtype == "f64" else torch.float32
    return torch.tensor(np.ascontiguousarray(a), dtype=t, device="cuda")


def host_input(a, dtype):
    """The values the oracle sees for an input of the given dtype."""
    a = np.asarray(a, dtype=np.float64)
    return a if dtype == "f64" else a.astype(np.float32).astype(np.float64)


def log_case(**kw):
    print("CASE " + " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def row_blocks(row_ptr, rows):
    """Indices of every block of the given block rows of a CSR pattern (for
    checking a subset of rows on its own)."""
    rows = np.unique(np.asarray(rows, dtype=np.int64))
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    starts = row_ptr[rows]
    lens = row_ptr[rows + 1] - starts
    first = np.cumsum(np.concatenate([[0], lens[:-1]]))
    return np.repeat(starts - first, lens) + np.arange(int(lens.sum()))
