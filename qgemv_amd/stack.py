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
pg_qgemv's products run on the matrix cores).  With a codebook table (batch 1,
fused) every group runs as one pg_rot_qgemv_table launch, the codes read
through that table.
"""
from __future__ import annotations

from . import _lib as L
from . import synth

ORDER = ("qkv", "o", "gu", "down")


class Stack:
    def __init__(self, shapes, layers: int, batch: int = 1, device: str = "cuda", x_dtype: int = L.PG_Q16,
                 fused: bool = True, carry: bool = False, split_above: int | None = None, table=None,
                 rate23: bool = False):
        import torch
        if table is not None and (not fused or batch != 1 or split_above is not None):
            raise ValueError("a codebook table runs on the fused batch-1 path only")
        # device int8 [8][256][4] codebook, or None for P8F v1's closed form;
        # rate23: the codes follow the rate-2/3 trellis (read through the table)
        if rate23 and table is None:
            raise ValueError("the rate-2/3 trellis is read through a codebook table")
        self.table = table
        if carry and not fused:
            raise ValueError("carried-state codes run on the fused path only")
        # random bytes are valid paths of both the per-block and the
        # carried-state trellis; carry selects how the stages read them
        self.cflag = (L.PG_FLAG_CARRY_STATE if carry else 0) | (L.PG_FLAG_RATE23 if rate23 else 0)
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

    def with_batch(self, batch: int, device: str = "cuda") -> "Stack":
        """A stack over the same device weights with its own activation and
        output buffers for `batch` rows."""
        import copy

        import torch
        other = copy.copy(self)
        other.batch = batch
        kmax = max(k for _, k in self.shapes.values())
        if self.x_dtype == L.PG_Q16:
            other.xrot = torch.zeros((batch, L.pg_q16_row_bytes(kmax)), dtype=torch.uint8, device=device)
        else:
            xt = torch.float32 if self.x_dtype == L.PG_F32 else torch.float16
            other.xrot = torch.empty((batch, kmax), dtype=xt, device=device)
        other.out = {site: torch.empty((batch, n), dtype=torch.float32, device=device)
                     for site, (n, _) in self.shapes.items()}
        other.h0 = torch.from_numpy(synth.activations_fp16(batch, self.raw_shapes["q"][1])).to(device)
        other.graph = None
        return other

    def launches(self, stream=None, h_in=None):
        """One token as a list of (kind, layer, site, call): kind "product"
        for a launch that reads the site's weights (pg_rot_qgemv or
        pg_qgemv), "rotate" for pg_fwht_rotate_ex; call() issues it."""
        b = self.batch
        out = []
        for layer in range(self.layers):
            for site in ORDER:
                n, k = self.shapes[site]
                c, s, g = self.codes[layer][site], self.scales[layer][site], self.signs[layer][site]
                y = self.out[site]
                first = site == "qkv" and layer == 0
                prev = {"qkv": "down", "o": "qkv", "gu": "o", "down": "gu"}[site]
                if first:
                    src, src_dt, ldx, flags = (h_in if h_in is not None else self.h0), L.PG_F16, k, 0
                else:
                    src, src_dt, ldx, flags = self.out[prev], L.PG_F32, self.shapes[prev][0], L.PG_FLAG_RMSNORM
                split = not self.fused or (self.split_above is not None and k > self.split_above and not first)
                if split:
                    xd = self.x_dtype if not self.fused else L.PG_Q16
                    out.append(("rotate", layer, site,
                                lambda src=src, src_dt=src_dt, ldx=ldx, g=g, k=k, flags=flags, xd=xd:
                                L.pg_fwht_rotate_ex(src, src_dt, ldx, self.xrot, xd, g, b, k, flags, stream)))
                    out.append(("product", layer, site,
                                lambda c=c, s=s, n=n, k=k, y=y, xd=xd:
                                L.pg_qgemv(c, s, n, k, self.xrot, xd, b, y, stream)))
                elif self.table is not None:
                    out.append(("product", layer, site,
                                lambda c=c, s=s, n=n, k=k, src=src, src_dt=src_dt, g=g, flags=flags, y=y:
                                L.pg_rot_qgemv_table(c, s, n, k, src, src_dt, g, self.table, flags | self.cflag, y,
                                                     stream)))
                else:
                    out.append(("product", layer, site,
                                lambda c=c, s=s, n=n, k=k, src=src, src_dt=src_dt, ldx=ldx, g=g, flags=flags, y=y:
                                L.pg_rot_qgemv(c, s, n, k, src, src_dt, ldx, g, flags | self.cflag, b, y, stream)))
        return out

    def token(self, stream=None, h_in=None):
        """Run one token through all layers; returns the last layer's d."""
        for _, _, _, call in self.launches(stream, h_in):
            call()
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

