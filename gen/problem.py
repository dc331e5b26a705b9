"""One seeded problem instance: every input tensor of the layer, available as
exact float64 slices on the host and as device tensors on the GPU.

Recipe (both sides):
  * x, dY ~ approximately N(0, 1);
  * router, gate and up weights ~ N(0, 1/d) (std 1/sqrt(fan_in), fan_in = d);
  * down weights ~ N(0, 1/I) (fan_in = I; I_s for the shared expert);
  * each tensor has its own Philox stream, element n uses counter n;
  * values are rounded once to fp32, then (for bf16 workloads) to bf16 (RNE);
  * skewed workloads add a per-expert logit bias b_e = ln p_rank(e) with
    p_r proportional to r^-s (Zipf), ranks given by a seeded Fisher-Yates
    permutation of the experts.
"""
import math

import numpy as np

from ._lib import host_fill, host_u32, device_fill, bf16_bits_to_f64

STREAMS = dict(x=1, w_router=2, w_gate=3, w_up=4, w_down=5, ws_gate=6, ws_up=7, ws_down=8, dy=9, perm=10)


class Problem:
    def __init__(self, dims):
        self.dims = dims
        self.bf16 = dims.prec != "f32"

    # ---- shapes and distributions -------------------------------------
    def shape(self, name):
        D = self.dims
        return {
            "x": (D.T, D.d), "dy": (D.T, D.d),
            "w_router": (D.E, D.d),
            "w_gate": (D.E, D.I, D.d), "w_up": (D.E, D.I, D.d), "w_down": (D.E, D.d, D.I),
            "ws_gate": (D.S, D.Is, D.d), "ws_up": (D.S, D.Is, D.d), "ws_down": (D.S, D.d, D.Is),
        }[name]

    def std(self, name):
        D = self.dims
        if name in ("x", "dy"):
            return 1.0
        if name == "w_down":
            return 1.0 / math.sqrt(D.I)
        if name == "ws_down":
            return 1.0 / math.sqrt(D.Is)
        return 1.0 / math.sqrt(D.d)

    def scale(self, name):
        # Irwin-Hall(8) has variance 8/12: sqrt(12/8) restores unit variance.
        return math.sqrt(1.5) * self.std(name)

    def numel(self, name):
        return int(np.prod(self.shape(name)))

    # ---- host side (exact float64 values of what is stored) ------------
    def host_flat(self, name, start, count):
        v = host_fill(start, count, self.dims.seed, STREAMS[name], self.scale(name), self.bf16)
        return bf16_bits_to_f64(v) if self.bf16 else v.astype(np.float64)

    def host(self, name):
        """Whole tensor as float64 (only for shapes that fit on the host)."""
        return self.host_flat(name, 0, self.numel(name)).reshape(self.shape(name))

    def host_rows(self, name, rows):
        """Selected rows of a 2-D tensor (x, dy, w_router) as float64 [len(rows)][cols]."""
        shp = self.shape(name)
        cols = shp[-1]
        out = np.empty((len(rows), cols), dtype=np.float64)
        for i, r in enumerate(rows):
            out[i] = self.host_flat(name, int(r) * cols, cols)
        return out

    def host_expert(self, name, e):
        """One expert's matrix of a stacked weight tensor, float64."""
        shp = self.shape(name)
        n = shp[1] * shp[2]
        return self.host_flat(name, int(e) * n, n).reshape(shp[1], shp[2])

    def host_expert_rows(self, name, e, rows):
        """Selected output rows of one expert's matrix, float64 [len(rows)][in]."""
        shp = self.shape(name)
        n = shp[1] * shp[2]
        out = np.empty((len(rows), shp[2]), dtype=np.float64)
        for i, r in enumerate(rows):
            out[i] = self.host_flat(name, int(e) * n + int(r) * shp[2], shp[2])
        return out

    def expert_permutation(self):
        """Fisher-Yates shuffle of range(E) driven by the 'perm' stream."""
        E = self.dims.E
        u = host_u32(0, max(E - 1, 0), self.dims.seed, STREAMS["perm"])
        pi = list(range(E))
        for step, i in enumerate(range(E - 1, 0, -1)):
            j = (int(u[step]) * (i + 1)) >> 32
            pi[i], pi[j] = pi[j], pi[i]
        return pi

    def logit_bias(self):
        """fp32 [E] Zipf logit bias, or None for unbiased workloads."""
        D = self.dims
        if D.zipf == 0.0:
            return None
        r = np.arange(1, D.E + 1, dtype=np.float64)
        p = r ** (-D.zipf)
        p /= p.sum()
        b = np.empty(D.E, dtype=np.float64)
        for rank, e in enumerate(self.expert_permutation()):
            b[e] = math.log(p[rank])
        return b.astype(np.float32)

    # ---- device side ----------------------------------------------------
    def device(self, name, device="cuda"):
        """Allocate a device tensor and fill it with the generator's values."""
        import torch
        dt = torch.bfloat16 if self.bf16 else torch.float32
        t = torch.empty(self.shape(name), dtype=dt, device=device)
        n = t.numel()
        if n:
            device_fill(t.data_ptr(), 0, n, self.dims.seed, STREAMS[name], self.scale(name), self.bf16,
                        torch.cuda.current_stream().cuda_stream)
        return t

    def device_bias(self, device="cuda"):
        import torch
        b = self.logit_bias()
        return None if b is None else torch.from_numpy(b).to(device)
