"""Device-side materialisation of synthetic logit rows (torch).  A pure bit
copy of the noise pool plus the bump writes, identical to the host copy in
synth.generators.materialize_rows_np."""
from __future__ import annotations

import numpy as np


class DeviceRows:
    def __init__(self, pool, device):
        import torch
        self.torch = torch
        self.pool = pool
        self.device = device
        bits = pool.bits
        tdt = torch.int16 if bits.dtype == np.uint16 else torch.int32
        host = torch.from_numpy(bits.view(np.int16 if bits.dtype == np.uint16 else np.int32))
        self.pool2 = torch.cat([host, host], dim=1).to(device).contiguous()
        self.tdt = tdt
        self.V = pool.V
        self.out_dtype = torch.bfloat16 if bits.dtype == np.uint16 else torch.float32

    def materialize(self, desc, out=None):
        torch = self.torch
        n = len(desc["idx"])
        win = self.pool2.unfold(1, self.V, 1)            # [rows, V+1, V] view
        idx = torch.from_numpy(np.asarray(desc["idx"], np.int64)).to(self.device)
        sh = torch.from_numpy(np.asarray(desc["shift"], np.int64)).to(self.device)
        rows = win[idx, sh]                              # gather copy [n, V]
        col = torch.from_numpy(np.asarray(desc["col"], np.int64)).to(self.device)
        bits = desc["bits"].view(np.int16 if desc["bits"].dtype == np.uint16 else np.int32)
        rows[torch.arange(n, device=self.device), col] = torch.from_numpy(bits.copy()).to(self.device)
        rows = rows.view(self.out_dtype)
        if out is not None:
            out.copy_(rows)
            return out
        return rows
