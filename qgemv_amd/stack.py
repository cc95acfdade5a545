"""Per-token driver for a synthetic linear stack (Qwen3-4B- or
Llama-3.1-8B-shaped layers) on one GPU.

Orchestration only: device buffers come from torch, every step is a
libpingala call on one stream.  Per layer, the four launch groups that
share an input are chained as
    x~ = R_qkv h        -> [q k v] = W~qkv x~
    x~ = R_o n16(q)     -> o        = W~o x~
    x~ = R_gu n16(o)    -> [g u]    = W~gu x~
    x~ = R_down n16(g)  -> d        = W~down x~ ,   h' = d
where n16 is the RMS normalisation with fp16 rounding; the first layer's
input is fp16 and is not normalised.  k, v and u are computed and stored but
not consumed.  The fused path (default) runs each group as one
pg_rot_qgemv launch (normalisation + rotation + product, batch 1..8); the
split path runs pg_fwht_rotate_ex then pg_qgemv (batch 1..8; from batch 2 on
pg_qgemv's products run on the matrix cores).
"""
from __future__ import annotations

from . import _lib as L
from . import synth

ORDER = ("qkv", "o", "gu", "down")


class Stack:
    def __init__(self, shapes, layers: int, batch: int = 1, device: str = "cuda", x_dtype: int = L.PG_Q16,
                 fused: bool = True, carry: bool = False, split_above: int | None = None):
        import torch
        if carry and not fused:
            raise ValueError("carried-state codes run on the fused path only")
        # random bytes are valid paths of both the per-block and the
        # carried-state trellis; carry selects how the stages read them
        self.cflag = L.PG_FLAG_CARRY_STATE if carry else 0
        # fused path: stages with k above this run as rotation + product
        # (pg_fwht_rotate_ex, pg_qgemv) instead of one pg_rot_qgemv
        if split_above is not None and carry:
            raise ValueError("carried-state codes run on the fused path only")
        self.split_above = split_above
        self.shapes = synth.merged_shapes(shapes)
        self.raw_shapes = shapes
        self.layers = layers
        self.batch = batch
        self.x_dtype = x_dtype
        self.codes, self.scales, self.signs = [], [], []
        self.bytes_per_token = 0
        for layer in range(layers):
            merged = synth.random_layer_merged(layer, shapes)
            c, s, g = {}, {}, {}
            for t, site in enumerate(ORDER):
                codes, scales = merged[site]
                c[site] = torch.from_numpy(codes).to(device)
                s[site] = torch.from_numpy(scales).to(device)
                g[site] = torch.from_numpy(synth.site_sign_bits(layer, t, self.shapes[site][1])).to(device)
                self.bytes_per_token += codes.nbytes + scales.nbytes
            self.codes.append(c)
            self.scales.append(s)
            self.signs.append(g)
        b = batch
        kmax = max(k for _, k in self.shapes.values())
        if x_dtype == L.PG_Q16:
            self.xrot = torch.zeros((b, L.pg_q16_row_bytes(kmax)), dtype=torch.uint8, device=device)
        else:
            xt = torch.float32 if x_dtype == L.PG_F32 else torch.float16
            self.xrot = torch.empty((b, kmax), dtype=xt, device=device)
        self.graph = None
        # fused path: one pg_rot_qgemv (normalisation + rotation + product)
        # per launch group
        self.fused = fused
        self.out = {site: torch.empty((b, n), dtype=torch.float32, device=device)
                    for site, (n, _) in self.shapes.items()}
        h = shapes["q"][1]
        self.h0 = torch.from_numpy(synth.activations_fp16(b, h)).to(device)

    def token(self, stream=None, h_in=None):
        """Run one token through all layers; returns the last layer's d."""
        if self.fused:
            return self._token_fused(stream, h_in)
        return self._token_split(stream, h_in)

    def _token_fused(self, stream=None, h_in=None):
        b = self.batch
        for layer in range(self.layers):
            for site in ORDER:
                n, k = self.shapes[site]
                if site == "qkv" and layer == 0:
                    src = h_in if h_in is not None else self.h0
                    L.pg_rot_qgemv(self.codes[layer][site], self.scales[layer][site], n, k, src, L.PG_F16, k,
                                   self.signs[layer][site], self.cflag, b, self.out[site], stream)
                    continue
                prev = {"qkv": "down", "o": "qkv", "gu": "o", "down": "gu"}[site]
                n_prev = self.shapes[prev][0]
                if self.split_above is not None and k > self.split_above:
                    L.pg_fwht_rotate_ex(self.out[prev], L.PG_F32, n_prev, self.xrot, L.PG_Q16, self.signs[layer][site],
                                        b, k, L.PG_FLAG_RMSNORM, stream)
                    L.pg_qgemv(self.codes[layer][site], self.scales[layer][site], n, k, self.xrot, L.PG_Q16, b,
                               self.out[site], stream)
                    continue
                L.pg_rot_qgemv(self.codes[layer][site], self.scales[layer][site], n, k, self.out[prev], L.PG_F32,
                               n_prev, self.signs[layer][site], L.PG_FLAG_RMSNORM | self.cflag, b, self.out[site],
                               stream)
        return self.out["down"]

    def _token_split(self, stream=None, h_in=None):
        b = self.batch
        for layer in range(self.layers):
            for site in ORDER:
                n, k = self.shapes[site]
                if site == "qkv":
                    if layer == 0:
                        src, src_dt, flags, ldx = (h_in if h_in is not None else self.h0), L.PG_F16, 0, k
                    else:
                        src, src_dt, flags, ldx = self.out["down"], L.PG_F32, L.PG_FLAG_RMSNORM, self.shapes["down"][0]
                else:
                    prev = {"o": "qkv", "gu": "o", "down": "gu"}[site]
                    src, src_dt, flags, ldx = self.out[prev], L.PG_F32, L.PG_FLAG_RMSNORM, self.shapes[prev][0]
                # the first k columns of each row of the previous output are the input
                L.pg_fwht_rotate_ex(src, src_dt, ldx, self.xrot, self.x_dtype, self.signs[layer][site], b, k, flags,
                                    stream)
                L.pg_qgemv(self.codes[layer][site], self.scales[layer][site], n, k, self.xrot, self.x_dtype,
                           b, self.out[site], stream)
        return self.out["down"]

    def capture(self):
        """Record one token's launches into a HIP graph (torch.cuda.CUDAGraph
        drives hipStreamBeginCapture on its own stream; the library launches
        on the current stream, which is that capture stream)."""
        import torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self.token()                      # warm the launch path outside capture
        torch.cuda.current_stream().wait_stream(s)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.token()
        self.graph = g
        return g

    def replay(self):
        self.graph.replay()
        return self.out["down"]

    def host_arrays(self, layer):
        """Numpy copies of one layer's codes, scales and signs (for checks)."""
        return ({s: self.codes[layer][s].cpu().numpy() for s in ORDER},
                {s: self.scales[layer][s].cpu().numpy() for s in ORDER},
                {s: self.signs[layer][s].cpu().numpy() for s in ORDER})

