"""Helpers shared by the GPU parity tests (comparison metrics, case logging)."""
import sys

import numpy as np
import torch


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def errs(got, ref):
    """max abs, max abs relative to max |ref|, RMSE and RMSE relative to rms(ref)."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    d = got - ref
    rms_ref = np.sqrt((ref ** 2).mean()) if ref.size else 0.0
    rmse = np.sqrt((d ** 2).mean()) if d.size else 0.0
    return dict(max_abs=float(np.abs(d).max(initial=0.0)),
                max_rel=float(np.abs(d).max(initial=0.0) / max(np.abs(ref).max(initial=0.0), 1e-30)),
                rmse=float(rmse), rel_rmse=float(rmse / max(rms_ref, 1e-30)))
