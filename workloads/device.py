"""Upload a generated workload to the device in the library's storage layouts.

Layout only (no arithmetic): x is the bf16 tensor of the drawn bits; the drawn A_a [K, r_a]
and B_a [r_a, N] go up as they are and the library packs them (lora_pack_adapter); W is
reordered into the packed form by the library's lora_pack_weight.
"""

from __future__ import annotations

import numpy as np
import torch

from precision_gemm_amd.ops import Adapters, LowpWeight, pack_weight


def bf16_tensor(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def upload(wl, device="cuda"):
    """Return (x, weight, adapters, ids) as device objects for workload ``wl``."""
    x = bf16_tensor(wl.x, device)
    q = torch.from_numpy(np.ascontiguousarray(wl.w_q)).to(device)
    s = torch.from_numpy(np.ascontiguousarray(wl.w_scale)).to(device)
    w = pack_weight(LowpWeight(wl.fmt, q, s))  # offline re-layout for the GEMM
    A = [bf16_tensor(a, device) for a in wl.A]
    B = [bf16_tensor(b, device) for b in wl.B]
    ad = Adapters(A, B, torch.from_numpy(np.asarray(wl.scale, np.float32)).to(device))
    ids = torch.from_numpy(np.asarray(wl.ids, np.int32)).to(device)
    return x, w, ad, ids
