"""CPU oracle for the Pingala-8 hot path, format P8F v1 (fp64, numpy).

TEST INFRASTRUCTURE ONLY.  Nothing in the product (the `qgemv_amd` package,
its HIP kernels or its C-ABI library) may import, call, link or execute this
module.  Only the test suite, `__graft_entry__.smoke()` and the CPU-baseline
leg of `bench.py` use it.  It shares no code with the library: every rule
below is written out again here from the method's description.

Sources.  The pages describe Pingala-8 in words only:
  [P1] "Pingala-8" landing page (ja), section 仕組み ("How it works"), with the
       same text in the zh landing page, section 原理: an Ungerboeck 8-state
       trellis code encodes groups of four weights in order; a small state
       carried from one group to the next picks the value set the next group
       may use; a random Hadamard rotation spreads out large weights before
       encoding; LDLQ rounding is used by the compressor.
  [P1-name] same page, section 名前の由来 ("Where the name comes from"): eight
       states over short three-syllable patterns, trellis labels after
       Ungerboeck.
  [P1-paper] same page, section 論文 ("Paper"): the title calls it small-state
       *coset* trellis coding.
  [P4] article "8 open models, 77-85% smaller: what 2-bit quantization costs
       and what it keeps", section "What 2-bit keeps": files carry per-block
       scales; batch-1 generation is dominated by reading the weights once per
       token.
The pages give no bit layout, codebook, block length or Hadamard size.  This
oracle follows format P8F v1, whose every choice is the plainest reading the
pages support (listed, with reasons, among the readings of the pages in the
design notes):
  * rotation: per 128-block, x~ = 2^-3.5 * H_128 * diag(sigma) * x, with H in
    Sylvester order and sigma the random signs of the input site;
  * a block is 128 consecutive rotated weights of one row = 32 groups of 4,
    with one fp16 scale (u16 bits); the trellis state is 0 at each block start;
  * state s in 0..7 is the three most recent branch bits, s' = ((s<<1)|u) & 7,
    u = bit 0 of the code byte;
  * z0(s) = bit 1 of s picks the value set A0 = {-7,-3,1,5} or
    A1 = {-5,-1,3,7} (units of the scale) for all four weights of the group;
    z1 = u ^ bit0(s) ^ bit2(s) picks the parity coset;
  * byte bits 1..3 are b0..b2, b3 = z1 ^ b0 ^ b1 ^ b2, bits 4..7 are e0..e3,
    p_j = 2 e_j + b_j and level_j = 4 p_j + 2 z0 - 7; weight = scale * level.
Products are plain fp64 sums.  The encoder is a Viterbi search for the
minimum-squared-error code sequence (LDLQ with an identity Hessian), with
fixed tie-breaks so that its output is unique.

Parity pins: every function here is checked in tests/test_oracle_*.py against
something other than itself (worked examples derived by hand, closed forms,
brute force on tiny inputs, invariants).  The one part the pages cannot pin
is coding quality (MSE); that is "parity unpinned" and only reported.
"""

from __future__ import annotations

import numpy as np

BLOCK = 128          # weights per scale block and per Hadamard block
GROUP = 4            # weights per trellis group (one code byte)
GROUPS_PER_BLOCK = BLOCK // GROUP
SCALE_C = 0.29       # encoder scale rule: s = fp16(c * rms(block))
FP16_MAX = 65504.0


# ---------------------------------------------------------------- rotation
def sylvester_hadamard(n: int) -> np.ndarray:
    """H[i, j] = (-1)^popcount(i & j), the Sylvester-ordered Hadamard matrix.

    Written entry by entry from its definition (no recursion, no FWHT)."""
    idx = np.arange(n)
    andm = idx[:, None] & idx[None, :]
    pop = np.zeros_like(andm)
    for bit in range(int(n).bit_length()):
        pop += (andm >> bit) & 1
    return np.where(pop % 2 == 0, 1.0, -1.0)


def signs_from_bits(sign_bits: np.ndarray, k: int) -> np.ndarray:
    """sigma_k = -1 where bit (k & 7) of byte (k >> 3) is set, else +1."""
    sign_bits = np.asarray(sign_bits, dtype=np.uint8)
    kk = np.arange(k)
    bits = (sign_bits[kk >> 3] >> (kk & 7)) & 1
    return np.where(bits == 1, -1.0, 1.0)


def rotation_block_matrix(sigma_block: np.ndarray) -> np.ndarray:
    """R_b = 2^-3.5 * H_128 * diag(sigma_b) for one 128-block ([P1] random
    Hadamard rotation; the normalisation makes R_b orthogonal)."""
    h = sylvester_hadamard(BLOCK)
    return (2.0 ** -3.5) * h * np.asarray(sigma_block, dtype=np.float64)[None, :]


def rotate(x: np.ndarray, sign_bits: np.ndarray) -> np.ndarray:
    """Apply the blockwise random-sign Hadamard rotation to the last axis.

    Used both for activations (x~ = R x) and for weight rows (w~_n = R w_n,
    i.e. W~ = W R^T), so that W~ x~ = W x.  Explicit 128x128 products in fp64."""
    x = np.asarray(x, dtype=np.float64)
    k = x.shape[-1]
    if k % BLOCK:
        raise ValueError("K must be a multiple of 128")
    sigma = signs_from_bits(sign_bits, k)
    out = np.empty_like(x)
    for b in range(k // BLOCK):
        rb = rotation_block_matrix(sigma[b * BLOCK:(b + 1) * BLOCK])
        out[..., b * BLOCK:(b + 1) * BLOCK] = x[..., b * BLOCK:(b + 1) * BLOCK] @ rb.T
    return out


# ------------------------------------------------------------ fp16 helpers
def fp16_rne(x) -> np.ndarray:
    """Round to IEEE binary16, round-to-nearest-even, back to fp64."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def fp16_bits_to_float(u16: np.ndarray) -> np.ndarray:
    return np.asarray(u16, dtype=np.uint16).view(np.float16).astype(np.float64)


def float_to_fp16_bits(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def bf16_rne_bits(x) -> np.ndarray:
    """fp32 -> bf16 bits with round-to-nearest-even (finite inputs)."""
    f = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (f + 0x7FFF + ((f >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_float(u16: np.ndarray) -> np.ndarray:
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ------------------------------------------------------------- the trellis
def next_state(s: int, u: int) -> int:
    """State = last three branch bits ([P1-name]: 8 states over 3-symbol
    patterns); the newest bit enters at bit 0."""
    return ((s << 1) | u) & 7


def z0_of_state(s: int) -> int:
    """Value set selected by the carried state ([P1]): A_{z0}."""
    return (s >> 1) & 1


def z1_of_branch(s: int, u: int) -> int:
    """Parity coset of the branch: z1 = u ^ bit0(s) ^ bit2(s)."""
    return u ^ (s & 1) ^ ((s >> 2) & 1)


def decode_group(byte: int, s: int) -> list[int]:
    """Four integer levels (units of the block scale) of one code byte read
    in state s."""
    u = byte & 1
    z0 = z0_of_state(s)
    z1 = z1_of_branch(s, u)
    b = [(byte >> 1) & 1, (byte >> 2) & 1, (byte >> 3) & 1]
    b.append(z1 ^ b[0] ^ b[1] ^ b[2])
    levels = []
    for j in range(4):
        e = (byte >> (4 + j)) & 1
        p = 2 * e + b[j]
        levels.append(4 * p + 2 * z0 - 7)
    return levels


def decode_block_levels(codes) -> list[int]:
    """Walk the trellis over one block's code bytes from state 0 and return
    all levels, group after group (scalar, serial: the definition)."""
    s = 0
    out: list[int] = []
    for byte in codes:
        byte = int(byte)
        out.extend(decode_group(byte, s))
        s = next_state(s, byte & 1)
    return out


def codebook_table() -> np.ndarray:
    """T[s][byte] = the four levels of `byte` read in state s (int8)."""
    t = np.zeros((8, 256, 4), dtype=np.int8)
    for s in range(8):
        for byte in range(256):
            t[s, byte] = decode_group(byte, s)
    return t


def decode_levels(codes: np.ndarray, carry: bool = False) -> np.ndarray:
    """Vectorised form of decode_block_levels for codes [..., K/4] (uint8).

    carry=False: the state restarts at 0 in every block (format P8F v1).
    carry=True: the variant whose state runs on from block to block along
    the row (decode_row_levels_carry is its definition).  Pinned against the
    scalar walks in the tests.  Returns int8 [..., K]."""
    c = np.asarray(codes, dtype=np.uint8)
    lead = c.shape[:-1]
    g = c.shape[-1]
    if g % GROUPS_PER_BLOCK:
        raise ValueError("K/4 must be a multiple of 32")
    if carry:
        c = c.reshape(lead + (1, g)).astype(np.int32)            # one trellis path per row
    else:
        c = c.reshape(lead + (g // GROUPS_PER_BLOCK, GROUPS_PER_BLOCK)).astype(np.int32)
    u = c & 1

    def prev(a, d):
        out = np.zeros_like(a)
        out[..., d:] = a[..., :-d]
        return out

    u1, u2, u3 = prev(u, 1), prev(u, 2), prev(u, 3)
    z0 = u2
    z1 = u ^ u1 ^ u3
    b0, b1, b2 = (c >> 1) & 1, (c >> 2) & 1, (c >> 3) & 1
    b3 = z1 ^ b0 ^ b1 ^ b2
    bs = [b0, b1, b2, b3]
    lv = np.empty(c.shape + (4,), dtype=np.int8)
    for j in range(4):
        e = (c >> (4 + j)) & 1
        lv[..., j] = 4 * (2 * e + bs[j]) + 2 * z0 - 7
    return lv.reshape(lead + (g * 4,))


def decode_weights(codes: np.ndarray, scales_u16: np.ndarray, carry: bool = False) -> np.ndarray:
    """Rotated-domain weights s * level as fp64 [..., K] (each value is exact
    in fp32 as well: an 11-bit scale times |level| <= 7)."""
    lv = decode_levels(codes, carry).astype(np.float64)
    s = fp16_bits_to_float(scales_u16)
    k = lv.shape[-1]
    return (lv.reshape(lv.shape[:-1] + (k // BLOCK, BLOCK)) * s[..., None]).reshape(lv.shape)


def levels_trellis_valid(levels: np.ndarray) -> bool:
    """Check that a level sequence (one block, 4*G values) is a trellis path:
    recover (z0, z1) of each group from its point, rebuild the branch bits and
    require the value set of every group to be the one its state allows."""
    lv = np.asarray(levels, dtype=np.int64).reshape(-1, 4)
    if not np.all(np.isin(lv, [-7, -5, -3, -1, 1, 3, 5, 7])):
        return False
    u_hist: list[int] = []
    for grp in lv:
        z0 = int(((grp[0] + 7) // 2) % 2)
        if not all(((v + 7) // 2) % 2 == z0 for v in grp):
            return False            # all four weights must share one value set
        p = (grp + 7 - 2 * z0) // 4
        z1 = int(np.sum(p % 2) % 2)
        um1 = u_hist[-1] if len(u_hist) >= 1 else 0
        um2 = u_hist[-2] if len(u_hist) >= 2 else 0
        um3 = u_hist[-3] if len(u_hist) >= 3 else 0
        if z0 != um2:
            return False
        u_hist.append(z1 ^ um1 ^ um3)
    return True


# ----------------------------------------------------------- scale rule
def block_scale_bits(w_rot_blocks: np.ndarray, c: float = SCALE_C) -> np.ndarray:
    """fp16 scale per block: s = fp16_RNE(min(c * rms, 65504)); 0 if rms is 0.

    The sum of squares runs sequentially over the 128 entries (a fixed order,
    so that every implementation of the rule rounds the same value)."""
    w = np.asarray(w_rot_blocks, dtype=np.float64)
    acc = np.zeros(w.shape[:-1], dtype=np.float64)
    for j in range(w.shape[-1]):
        acc = acc + w[..., j] * w[..., j]
    rms = np.sqrt(acc / w.shape[-1])
    val = np.minimum(c * rms, FP16_MAX)
    return float_to_fp16_bits(val)


# ------------------------------------------------------- Viterbi encoder
def _point_tables():
    """For each (z0, z1): the 128 bytes of that coset in increasing order and
    their 4-D level points.  The byte <-> point map of a state depends only
    on (z0, z1), so states sharing them share the table."""
    tabs = {}
    for z0 in (0, 1):
        for z1 in (0, 1):
            # any state with these (z0, z1) for branch u: pick s with
            # bit1 = z0, and u chosen so that z1 matches with bit0 = bit2 = 0
            s = z0 << 1
            u = z1
            bytes_ = np.array([b for b in range(256) if (b & 1) == u], dtype=np.int64)
            pts = np.array([decode_group(int(b), s) for b in bytes_], dtype=np.float64)
            tabs[(z0, z1)] = (bytes_, pts)
    return tabs


_TABS = None


def _tabs():
    global _TABS
    if _TABS is None:
        _TABS = _point_tables()
    return _TABS


def branch_metrics(w_groups: np.ndarray, s_val: np.ndarray):
    """Distortion of the nearest point of every coset for every group.

    w_groups [nb, G, 4] fp64, s_val [nb].  Returns dict (z0, z1) ->
    (metric [nb, G], byte [nb, G]).  Brute force over all 128 points of the
    coset, each distortion evaluated as ((d0^2 + d1^2) + d2^2) + d3^2 with
    d_j = w_j - s * level_j; the smallest byte wins ties (first minimum in
    ascending byte order)."""
    out = {}
    for key, (bytes_, pts) in _tabs().items():
        # pts [128, 4] in ascending byte order; distortion per point
        d = w_groups[:, :, None, :] - s_val[:, None, None, None] * pts[None, None, :, :]
        sq = d * d
        m = ((sq[..., 0] + sq[..., 1]) + sq[..., 2]) + sq[..., 3]     # [nb, G, 128]
        arg = np.argmin(m, axis=2)                                    # first minimum
        best = np.take_along_axis(m, arg[..., None], axis=2)[..., 0]
        out[key] = (best, bytes_[arg])
    return out


def viterbi_encode(w_rot: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """Minimum-squared-error trellis path for each block.

    w_rot [nb, 4G] fp64 rotated weights, scale_bits [nb] u16.  G is free (32
    for real blocks; tests use short blocks).  Start in state 0, free end
    state.  Tie-breaks (strict < in ascending order): predecessor s'>>1 over
    (s'>>1)|4, smaller byte among equally near points, smaller end state.
    A zero scale codes every group as byte 0."""
    w = np.asarray(w_rot, dtype=np.float64)
    nb = w.shape[0]
    g = w.shape[1] // 4
    wg = w.reshape(nb, g, 4)
    s_val = fp16_bits_to_float(scale_bits)
    bm = branch_metrics(wg, s_val)
    inf = np.inf
    metric = np.full((nb, 8), inf)
    metric[:, 0] = 0.0
    back_prev = np.zeros((nb, g, 8), dtype=np.int8)     # predecessor state
    back_byte = np.zeros((nb, g, 8), dtype=np.int16)    # byte on that branch
    for t in range(g):
        new = np.full((nb, 8), inf)
        for sn in range(8):
            u = sn & 1
            for cand in (sn >> 1, (sn >> 1) | 4):
                key = (z0_of_state(cand), z1_of_branch(cand, u))
                m_b, byte_b = bm[key]
                tot = metric[:, cand] + m_b[:, t]
                better = tot < new[:, sn]
                new[:, sn] = np.where(better, tot, new[:, sn])
                back_prev[:, t, sn] = np.where(better, cand, back_prev[:, t, sn])
                # the coset table's bytes carry bit 0 = z1; on this branch the
                # byte's bit 0 is the branch bit u (bits 1..7 pick the point)
                byte_u = (byte_b[:, t] & 0xFE) | u
                back_byte[:, t, sn] = np.where(better, byte_u, back_byte[:, t, sn])
        metric = new
    end = np.argmin(metric, axis=1)        # first minimum = smaller state on ties
    codes = np.zeros((nb, g), dtype=np.uint8)
    st = end.copy()
    rows = np.arange(nb)
    for t in range(g - 1, -1, -1):
        codes[:, t] = back_byte[rows, t, st].astype(np.uint8)
        st = back_prev[rows, t, st].astype(np.int64)
    codes[s_val == 0] = 0
    return codes


def block_distortion(w_rot: np.ndarray, codes: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """Squared error of each block's decoded path (fp64)."""
    lv = np.stack([np.array(decode_block_levels(c), dtype=np.float64) for c in codes])
    s = fp16_bits_to_float(scale_bits)[:, None]
    d = np.asarray(w_rot, dtype=np.float64) - s * lv
    return np.sum(d * d, axis=1)


def exhaustive_encode_bytes(w_rot_row: np.ndarray, scale_bits: int):
    """All 256^G byte strings of a short block (G <= 3), each decoded through
    the state table (state = last three branch bits, 0 at the start).
    Returns (min distortion, first minimising string in lexicographic order,
    group 0 most significant)."""
    w = np.asarray(w_rot_row, dtype=np.float64)
    g = len(w) // 4
    if g > 3:
        raise ValueError("exhaustive byte search is for G <= 3")
    s = float(fp16_bits_to_float(np.array([scale_bits]))[0])
    table = codebook_table().astype(np.float64)           # [8, 256, 4]
    tail = g - 1
    rest = np.arange(256 ** tail, dtype=np.int64)
    rest_bytes = [(rest >> (8 * (tail - 1 - t))) & 0xFF for t in range(tail)]
    best, best_codes = np.inf, None
    for b0 in range(256):                                  # lexicographic order
        bytes_ = [np.full(rest.shape, b0, dtype=np.int64)] + rest_bytes
        st = np.zeros(rest.shape, dtype=np.int64)
        acc = np.zeros(rest.shape)
        for t in range(g):
            lv = table[st, bytes_[t]]                      # [n, 4]
            d = w[4 * t:4 * t + 4][None, :] - s * lv
            sq = d * d
            acc = acc + (((sq[:, 0] + sq[:, 1]) + sq[:, 2]) + sq[:, 3])
            st = ((st << 1) | (bytes_[t] & 1)) & 7
        i = int(np.argmin(acc))
        if acc[i] < best:
            best = float(acc[i])
            best_codes = [int(bytes_[t][i]) for t in range(g)]
    return best, best_codes


def exhaustive_encode_paths(w_rot_row: np.ndarray, scale_bits: int) -> float:
    """Minimum distortion over all 2^G branch paths, each group taking the
    nearest point of its coset by brute force (G <= 12)."""
    w = np.asarray(w_rot_row, dtype=np.float64)
    g = len(w) // 4
    s = float(fp16_bits_to_float(np.array([scale_bits]))[0])
    tabs = _tabs()
    # nearest-point distortion per group per coset
    near = {}
    for key, (_, pts) in tabs.items():
        d = w.reshape(g, 1, 4) - s * pts[None, :, :]
        near[key] = np.min(np.sum(d * d, axis=2), axis=1)
    best = np.inf
    for path in range(1 << g):
        st = 0
        acc = 0.0
        for t in range(g):
            u = (path >> t) & 1
            acc += near[(z0_of_state(st), z1_of_branch(st, u))][t]
            st = next_state(st, u)
        best = min(best, acc)
    return best


_CLIB = None


def _c_lib():
    """The oracle's plain-C twin of viterbi_encode (oracle/viterbi_ref.c)."""
    global _CLIB
    if _CLIB is None:
        import ctypes
        import os
        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liboracle_p8f.so")
        if not os.path.exists(path):
            from . import build_oracle
            build_oracle.build()
        lib = ctypes.CDLL(path)
        lib.p8f_oracle_viterbi.restype = ctypes.c_int
        lib.p8f_oracle_viterbi.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                           ctypes.c_int, ctypes.c_void_p]
        _CLIB = lib
    return _CLIB


def viterbi_encode_c(w_rot: np.ndarray, scale_bits: np.ndarray, threads: int = 0) -> np.ndarray:
    """Same search as viterbi_encode, run by the C twin (bit-identical
    metrics: same brute force, same evaluation order, no fused multiply-add).
    Blocks are split over `threads` Python threads (ctypes drops the GIL)."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    w = np.ascontiguousarray(w_rot, dtype=np.float64)
    sb = np.ascontiguousarray(scale_bits, dtype=np.uint16)
    nb, g4 = w.shape
    g = g4 // 4
    codes = np.zeros((nb, g), dtype=np.uint8)
    lib = _c_lib()
    nt = threads or min(16, os.cpu_count() or 1)
    bounds = np.linspace(0, nb, nt + 1).astype(np.int64)

    def run(i):
        a, b = int(bounds[i]), int(bounds[i + 1])
        if b > a:
            rc = lib.p8f_oracle_viterbi(w[a:b].ctypes.data, sb[a:b].ctypes.data, b - a, g,
                                        codes[a:b].ctypes.data)
            if rc != 0:
                raise RuntimeError("oracle viterbi failed")

    with ThreadPoolExecutor(nt) as ex:
        list(ex.map(run, range(nt)))
    return codes


def encode_matrix(w: np.ndarray, sign_bits: np.ndarray, c: float = SCALE_C,
                  chunk_blocks: int = 2048, use_c: bool = True):
    """Offline compression of W [N][K] (fp32 values, original domain):
    rotate each row, set each block's fp16 scale, Viterbi-encode.
    Returns codes u8 [N][K/4] and scale bits u16 [N][K/128]."""
    w = np.asarray(w, dtype=np.float32).astype(np.float64)
    n, k = w.shape
    nbk = k // BLOCK
    codes = np.empty((n, k // 4), dtype=np.uint8)
    scales = np.empty((n, nbk), dtype=np.uint16)
    if use_c:
        chunk_blocks = max(chunk_blocks, 65536)
    rows_per_chunk = max(1, chunk_blocks // nbk)
    for r0 in range(0, n, rows_per_chunk):
        r1 = min(n, r0 + rows_per_chunk)
        wr = rotate(w[r0:r1], sign_bits).reshape(-1, BLOCK)
        sb = block_scale_bits(wr, c)
        cb = viterbi_encode_c(wr, sb) if use_c else viterbi_encode(wr, sb)
        codes[r0:r1] = cb.reshape(r1 - r0, k // 4)
        scales[r0:r1] = sb.reshape(r1 - r0, nbk)
    return codes, scales


# -------------------------------------------------------------- products
def gemv_ref(codes: np.ndarray, scales_u16: np.ndarray, x_rot: np.ndarray, carry: bool = False) -> np.ndarray:
    """y[b][n] = sum_blk s[n][blk] * sum_{k in blk} level[n][k] * x~[b][k], fp64.

    x_rot [B][K] (any float dtype; taken exactly).  Returns fp64 [B][N].
    carry selects the carried-state variant's levels."""
    lv = decode_levels(codes, carry).astype(np.float64)       # [N, K]
    n, k = lv.shape
    x = np.asarray(x_rot, dtype=np.float64).reshape(-1, k)
    s = fp16_bits_to_float(scales_u16)                          # [N, nb]
    part = np.einsum("nbk,mbk->mnb", lv.reshape(n, k // BLOCK, BLOCK),
                     x.reshape(x.shape[0], k // BLOCK, BLOCK))  # per-block dots
    return np.einsum("mnb,nb->mn", part, s)


def gemm_ref(codes, scales_u16, x_rot):
    """Same product for M activation rows (prompt processing): Y [M][N]."""
    return gemv_ref(codes, scales_u16, x_rot)


def gemv_rows_ref(codes_rows, scales_rows, x_rot):
    """gemv_ref restricted to selected rows (for sampled checks at full size)."""
    return gemv_ref(codes_rows, scales_rows, x_rot)


# ------------------------------------------------------- activation chain
def rmsnorm16(v: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """fp16_RNE(v / sqrt(mean(v^2) + eps)) over the last axis (fp64 math).

    The normalisation that keeps activations in fp16 range between the
    layers of a synthetic linear stack (the pages' decoder layers feed each
    matrix's output onward; norm layers sit between them)."""
    v = np.asarray(v, dtype=np.float64)
    r = np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)
    return fp16_rne(v / r)


# ------------------------------------------- variant: state carried on
# The landing page's "Paper" section places the format in the small-state
# coset-trellis design space; one point of that space keeps the trellis
# state running from block to block along a row instead of restarting it at
# 0 in every 128-block.  Scales stay per block; a zero-scale block is still
# coded as 32 zero bytes (which leaves the state at 0 for the next block).
def decode_row_levels_carry(codes_row) -> list[int]:
    """Definition of the variant's decode: one scalar trellis walk over all
    code bytes of a row from state 0, never reset."""
    s = 0
    out: list[int] = []
    for byte in codes_row:
        byte = int(byte)
        out.extend(decode_group(byte, s))
        s = next_state(s, byte & 1)
    return out


def viterbi_encode_row_carry(w_rot_blocks: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """Minimum-squared-error path through all blocks of one row with the
    state carried on: w_rot_blocks [nb, 4G] fp64 (G = 32 for real blocks),
    scale_bits [nb] u16.  One Viterbi over nb * G steps from state 0 with a
    free end state; block b's branch metrics use its own scale.  In a
    zero-scale block the only branch is byte 0 (u = 0, point 0) at no cost.
    Tie-breaks as in viterbi_encode.  Returns codes [nb, G]."""
    w = np.asarray(w_rot_blocks, dtype=np.float64)
    nb, g = w.shape[0], w.shape[1] // 4
    s_val = fp16_bits_to_float(np.asarray(scale_bits, dtype=np.uint16))
    bm = branch_metrics(w.reshape(nb, g, 4), s_val)
    inf = np.inf
    metric = np.full(8, inf)
    metric[0] = 0.0
    steps = nb * g
    back_prev = np.zeros((steps, 8), dtype=np.int64)
    back_byte = np.zeros((steps, 8), dtype=np.int64)
    for b in range(nb):
        for t in range(g):
            new = np.full(8, inf)
            i = b * g + t
            for sn in range(8):
                u = sn & 1
                for cand in (sn >> 1, (sn >> 1) | 4):
                    if s_val[b] == 0:
                        if u != 0:
                            continue
                        m_t, byte = 0.0, 0
                    else:
                        m_b, byte_b = bm[(z0_of_state(cand), z1_of_branch(cand, u))]
                        m_t, byte = m_b[b, t], (int(byte_b[b, t]) & 0xFE) | u
                    tot = metric[cand] + m_t
                    if tot < new[sn]:
                        new[sn] = tot
                        back_prev[i, sn] = cand
                        back_byte[i, sn] = byte
            metric = new
    st = int(np.argmin(metric))
    out = np.zeros(steps, dtype=np.uint8)
    for i in range(steps - 1, -1, -1):
        out[i] = back_byte[i, st]
        st = int(back_prev[i, st])
    return out.reshape(nb, g)


def row_distortion_carry(w_rot_blocks: np.ndarray, codes_row_blocks: np.ndarray, scale_bits: np.ndarray) -> float:
    """Squared error of a row's decoded path in the carried-state variant."""
    w = np.asarray(w_rot_blocks, dtype=np.float64)
    lv = np.array(decode_row_levels_carry(np.asarray(codes_row_blocks).reshape(-1)), dtype=np.float64)
    s = np.repeat(fp16_bits_to_float(np.asarray(scale_bits, dtype=np.uint16)), w.shape[1])
    d = w.reshape(-1) - s * lv
    return float(np.sum(d * d))


def exhaustive_encode_paths_carry(w_rot_blocks: np.ndarray, scale_bits) -> float:
    """Minimum distortion over all 2^(nb G) branch paths of a short row in
    the carried-state variant, each group taking the nearest point of its
    coset by brute force (nb G <= 12; no zero-scale blocks)."""
    w = np.asarray(w_rot_blocks, dtype=np.float64)
    nb, g = w.shape[0], w.shape[1] // 4
    near = []
    for b in range(nb):
        sv = float(fp16_bits_to_float(np.array([scale_bits[b]], dtype=np.uint16))[0])
        nb_near = {}
        for key, (_, pts) in _tabs().items():
            d = w[b].reshape(g, 1, 4) - sv * pts[None, :, :]
            nb_near[key] = np.min(np.sum(d * d, axis=2), axis=1)
        near.append(nb_near)
    best = np.inf
    for path in range(1 << (nb * g)):
        st, acc = 0, 0.0
        for i in range(nb * g):
            u = (path >> i) & 1
            acc += near[i // g][(z0_of_state(st), z1_of_branch(st, u))][i % g]
            st = next_state(st, u)
        best = min(best, acc)
    return best


def encode_matrix_carry(w: np.ndarray, sign_bits: np.ndarray, c: float = SCALE_C):
    """Offline compression in the carried-state variant: rotate, per-block
    scales (the same rule), one Viterbi per row.  Returns codes u8 [N][K/4]
    and scale bits u16 [N][K/128]."""
    w = np.asarray(w, dtype=np.float32).astype(np.float64)
    n, k = w.shape
    nbk = k // BLOCK
    wr = rotate(w, sign_bits).reshape(n, nbk, BLOCK)
    scales = block_scale_bits(wr.reshape(-1, BLOCK), c).reshape(n, nbk)
    codes = np.empty((n, k // 4), dtype=np.uint8)
    for r in range(n):
        codes[r] = viterbi_encode_row_carry(wr[r], scales[r]).reshape(-1)
    return codes, scales


# ------------------------------------- variant: table-driven codebook
# The landing page's "Paper" section places the format in the small-state
# coset-trellis design space.  Its two halves are separable: the trellis
# fixes the branch bit of a byte (u = bit 0) and the state that follows, the
# codebook fixes the 4-D point a byte names in a state.  A table T[s][byte]
# of four int8 levels (units of the block scale, 8 x 256 x 4 bytes) holds any
# such codebook: P8F v1's closed-form rule is one table (codebook_table), a
# non-uniform or learned value set another.  Trellis, scales, block length
# and rotation stay as in P8F v1; the state restarts at 0 in every block
# unless carry is asked for.
def decode_block_levels_table(codes, table) -> list[int]:
    """Definition of the table decode: one scalar walk over one block's code
    bytes from state 0; each group's four levels are T[s][byte]."""
    t = np.asarray(table, dtype=np.int8).reshape(8, 256, 4)
    s = 0
    out: list[int] = []
    for byte in codes:
        byte = int(byte)
        out.extend(int(v) for v in t[s, byte])
        s = next_state(s, byte & 1)
    return out


def trellis_states(codes: np.ndarray, carry: bool = False, rate23: bool = False) -> np.ndarray:
    """The state each code byte of codes [..., K/4] is read in, zero before
    the block's (with carry: the row's) start.  P8F v1: the three previous
    branch bits, the newest at bit 0.  Rate 2/3 (the variant below): the
    previous byte's two branch bits at bits 0, 1 and the branch bit u0 of
    the byte before it at bit 2 (s' = ((s << 2) | u) & 7 unrolled).  Pinned
    against the scalar walks in the tests."""
    c = np.asarray(codes, dtype=np.uint8)
    lead, g = c.shape[:-1], c.shape[-1]
    if g % GROUPS_PER_BLOCK:
        raise ValueError("K/4 must be a multiple of 32")
    shape = lead + (1, g) if carry else lead + (g // GROUPS_PER_BLOCK, GROUPS_PER_BLOCK)
    c = c.reshape(shape).astype(np.int32)
    s = np.zeros_like(c)
    if rate23:
        s[..., 1:] |= c[..., :-1] & 3
        s[..., 2:] |= (c[..., :-2] & 1) << 2
    else:
        u = c & 1
        for d in (1, 2, 3):                  # branch bit d groups back -> state bit d - 1
            s[..., d:] |= u[..., :-d] << (d - 1)
    return s.reshape(lead + (g,))


def decode_levels_table(codes: np.ndarray, table: np.ndarray, carry: bool = False,
                        rate23: bool = False) -> np.ndarray:
    """Levels of codes [..., K/4] under the table T [8][256][4] int8: the
    group read in state s as byte c takes T[s][c]; the states follow P8F
    v1's trellis, or the rate-2/3 one.  Returns int8 [..., K]."""
    c = np.asarray(codes, dtype=np.uint8)
    t = np.asarray(table, dtype=np.int8).reshape(8, 256, 4)
    s = trellis_states(c, carry, rate23)
    return t[s, c].reshape(c.shape[:-1] + (c.shape[-1] * 4,))


def decode_weights_table(codes: np.ndarray, scales_u16: np.ndarray, table: np.ndarray,
                         carry: bool = False, rate23: bool = False) -> np.ndarray:
    """Rotated-domain weights s * T-level as fp64 [..., K] (exact in fp32 as
    well: an 11-bit scale times an 8-bit level)."""
    lv = decode_levels_table(codes, table, carry, rate23).astype(np.float64)
    s = fp16_bits_to_float(scales_u16)
    k = lv.shape[-1]
    return (lv.reshape(lv.shape[:-1] + (k // BLOCK, BLOCK)) * s[..., None]).reshape(lv.shape)


def gemv_table_ref(codes: np.ndarray, scales_u16: np.ndarray, table: np.ndarray, x_rot: np.ndarray,
                   carry: bool = False, rate23: bool = False) -> np.ndarray:
    """y[b][n] = sum_blk s[n][blk] * sum_{k in blk} T-level[n][k] * x~[b][k] in
    fp64, x_rot [B][K].  Returns fp64 [B][N]."""
    lv = decode_levels_table(codes, table, carry, rate23).astype(np.float64)
    n, k = lv.shape
    x = np.asarray(x_rot, dtype=np.float64).reshape(-1, k)
    s = fp16_bits_to_float(scales_u16)
    part = np.einsum("nbk,mbk->mnb", lv.reshape(n, k // BLOCK, BLOCK),
                     x.reshape(x.shape[0], k // BLOCK, BLOCK))
    return np.einsum("mnb,nb->mn", part, s)


# ------------------------------------- variant: rate-2/3 trellis, 8 cosets
# The landing page's "Where the name comes from" section: eight states over
# short patterns, labels in Ungerboeck's manner; "Paper" names the family a
# small-state coset trellis.  P8F v1 spends one branch bit per group (rate
# 1/2 over 4 cosets of 128 points); this variant spends two (rate 2/3, four
# branches per state) over 8 cosets of 64 points of the same 512-point set
# (four coordinates, levels 4 p + 2 z0 - 7 with p = 2 e + b), still 8 bits a
# group.  The set is split in Ungerboeck's way along the chain
# A0|A1 (z0: the value set) / D4 parity (z1 = b0^b1^b2^b3) / the RZ4 split
# (z2 = b0^b1).  Byte bits 0, 1 are the branch u = (u0, u1); bits 2, 3 are
# b0, b2 (b1 = b0 ^ z2, b3 = b2 ^ z1 ^ z2); bits 4..7 are e0..e3.  The state
# is a shift register of the branch bits, s' = ((s << 2) | u) & 7, 0 at each
# block start.  Ungerboeck's rules fix the labels: the four branches that
# leave a state, and the four that enter one, take the four cosets of one
# value set, z0 = bit 0 of s, and (z1, z2) = (u0 ^ bit 1 of s, u1 ^ bit 2 of
# s) gives both groups of four distinct cosets.
def next_state_r23(s: int, u: int) -> int:
    return ((s << 2) | u) & 7


def coset_r23(s: int, u: int) -> tuple[int, int, int]:
    """(z0, z1, z2) of the branch u out of state s."""
    return s & 1, (u & 1) ^ ((s >> 1) & 1), ((u >> 1) & 1) ^ ((s >> 2) & 1)


def decode_group_r23(byte: int, s: int) -> list[int]:
    """Four integer levels of one code byte read in state s (rate 2/3)."""
    z0, z1, z2 = coset_r23(s, byte & 3)
    b0, b2 = (byte >> 2) & 1, (byte >> 3) & 1
    b = [b0, b0 ^ z2, b2, b2 ^ z1 ^ z2]
    return [4 * (2 * ((byte >> (4 + j)) & 1) + b[j]) + 2 * z0 - 7 for j in range(4)]


def codebook_table_r23() -> np.ndarray:
    """T[s][byte] = the four levels of `byte` read in state s (rate 2/3, int8):
    with the rate-2/3 states, the table decode reproduces this variant."""
    t = np.zeros((8, 256, 4), dtype=np.int8)
    for s in range(8):
        for byte in range(256):
            t[s, byte] = decode_group_r23(byte, s)
    return t


def decode_block_levels_r23(codes) -> list[int]:
    """Definition of the rate-2/3 decode: one scalar walk over one block's
    bytes from state 0."""
    s = 0
    out: list[int] = []
    for byte in codes:
        byte = int(byte)
        out.extend(decode_group_r23(byte, s))
        s = next_state_r23(s, byte & 3)
    return out


def coset_of_levels(grp) -> tuple[int, int, int]:
    """(z0, z1, z2) of a 4-D point of the 512-point set (levels odd, |l| <= 7,
    all four in one value set); ValueError otherwise."""
    lv = [int(v) for v in grp]
    if any(v not in (-7, -5, -3, -1, 1, 3, 5, 7) for v in lv):
        raise ValueError("level outside the 8-level alphabet")
    z0s = {((v + 7) // 2) % 2 for v in lv}
    if len(z0s) != 1:
        raise ValueError("the four levels are not in one value set")
    z0 = z0s.pop()
    b = [((v + 7 - 2 * z0) // 4) % 2 for v in lv]
    return z0, b[0] ^ b[1] ^ b[2] ^ b[3], b[0] ^ b[1]


def levels_trellis_valid_r23(levels) -> bool:
    """A level sequence (one block) is a rate-2/3 path: every group's coset
    is one that a branch out of the current state carries; the branch it
    takes is then unique and fixes the next state."""
    lv = np.asarray(levels, dtype=np.int64).reshape(-1, 4)
    s = 0
    for grp in lv:
        try:
            z = coset_of_levels(grp)
        except ValueError:
            return False
        us = [u for u in range(4) if coset_r23(s, u) == z]
        if len(us) != 1:
            return False
        s = next_state_r23(s, us[0])
    return True


def _coset_points_r23():
    """For each coset (z0, z1, z2): its 64 points as (bytes without the
    branch bits, levels [64][4]), the byte's bits 2..7 ascending."""
    out = {}
    for z0 in range(2):
        for z1 in range(2):
            for z2 in range(2):
                # a state and branch that carry this coset: s = z0 (bits 1, 2 zero), u = (z1, z2)
                s, u = z0, z1 | (z2 << 1)
                assert coset_r23(s, u) == (z0, z1, z2)
                bytes_ = np.array([(hi << 2) | u for hi in range(64)], dtype=np.int64)
                pts = np.array([decode_group_r23(int(c), s) for c in bytes_], dtype=np.float64)
                out[(z0, z1, z2)] = (bytes_ >> 2, pts)
    return out


def viterbi_encode_r23(w_rot: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """Minimum-squared-error rate-2/3 path per block: w_rot [nb, 4G] fp64,
    scale_bits [nb] u16.  Per group and coset the nearest of its 64 points by
    brute force (lowest byte on ties); then a Viterbi over 8 states from state
    0 with a free end state (predecessors tried in increasing state and
    branch order, strict improvement, lowest final state).  A zero-scale
    block codes as bytes 0 (the all-zero branch sequence, any point)."""
    w = np.asarray(w_rot, dtype=np.float64)
    nb, g = w.shape[0], w.shape[1] // 4
    sv = fp16_bits_to_float(np.asarray(scale_bits, dtype=np.uint16))
    cos = _coset_points_r23()
    out = np.zeros((nb, g), dtype=np.uint8)
    for b in range(nb):
        if sv[b] == 0:
            continue
        near = {}
        for z, (hi, pts) in cos.items():
            d = w[b].reshape(g, 1, 4) - sv[b] * pts[None, :, :]
            dist = np.sum(d * d, axis=2)                 # [g, 64]
            i = np.argmin(dist, axis=1)                  # first minimum: lowest byte
            near[z] = (dist[np.arange(g), i], hi[i])
        metric = np.full(8, np.inf)
        metric[0] = 0.0
        back = np.zeros((g, 8, 2), dtype=np.int64)       # (previous state, byte)
        for t in range(g):
            new = np.full(8, np.inf)
            for sp in range(8):
                if metric[sp] == np.inf:
                    continue
                for u in range(4):
                    z = coset_r23(sp, u)
                    tot = metric[sp] + near[z][0][t]
                    sn = next_state_r23(sp, u)
                    if tot < new[sn]:
                        new[sn] = tot
                        back[t, sn] = (sp, (int(near[z][1][t]) << 2) | u)
            metric = new
        st = int(np.argmin(metric))
        for t in range(g - 1, -1, -1):
            out[b, t] = back[t, st, 1]
            st = int(back[t, st, 0])
    return out


def block_distortion_r23(w_rot: np.ndarray, codes: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """Squared error per block of the rate-2/3 decode of codes [nb, G]."""
    w = np.asarray(w_rot, dtype=np.float64)
    sv = fp16_bits_to_float(np.asarray(scale_bits, dtype=np.uint16))
    out = np.zeros(w.shape[0])
    for b in range(w.shape[0]):
        lv = np.array(decode_block_levels_r23(codes[b]), dtype=np.float64)
        d = w[b] - sv[b] * lv
        out[b] = float(np.sum(d * d))
    return out


def exhaustive_encode_r23(w_rot_row: np.ndarray, scale_bits: int) -> float:
    """Minimum distortion over every byte string of a short block (256^G
    strings, G <= 3), each decoded by the scalar walk: the brute-force
    optimum that the Viterbi must reach."""
    w = np.asarray(w_rot_row, dtype=np.float64)
    g = w.shape[0] // 4
    sv = float(fp16_bits_to_float(np.array([scale_bits], dtype=np.uint16))[0])
    best = np.inf
    for idx in range(256 ** g):
        codes = [(idx >> (8 * t)) & 255 for t in range(g)]
        d = w - sv * np.array(decode_block_levels_r23(codes), dtype=np.float64)
        best = min(best, float(np.sum(d * d)))
    return best


# ------------------------------------------- LDLQ with a proxy Hessian
# The landing page's "How it works" section names LDLQ as the compressor's
# rounding: each coded unit's error is passed on, through the Hessian of the
# layer's inputs, to the units not yet coded.  Here the unit is the 128-block
# (the trellis restarts per block, so a block's codes are final only when its
# Viterbi ends): with H~ = R H R^T the Hessian in the rotated basis, and
# H~ = U D U^T (U unit upper block-triangular, D block-diagonal, blocks of
# 128), block j is coded against the target
#     T_j = W~_j + sum_{c < 128 j} (W~ - What)[:, c] * U[c, block j]
# (its scale from T_j by the usual rule), so that the proxy loss
# tr(E H~ E^T), E = What - W~, equals sum_j tr(eta_j D_j eta_j^T) with eta_j
# = What_j - T_j the block's own rounding error.  H = I gives U = I and the
# plain encoder.  The feedback sum runs over c in increasing order, one
# rounding per product and per addition (fp64), the order the library's
# encoders use.
def rotate_hessian(h: np.ndarray, sign_bits: np.ndarray) -> np.ndarray:
    """H~ = R H R^T for the block rotation R of the input site (fp64)."""
    hr = rotate(np.asarray(h, dtype=np.float64), sign_bits)     # H R^T
    return rotate(np.ascontiguousarray(hr.T), sign_bits)        # R (H R^T)^T R^T = R H R^T (H symmetric)


def block_udu(h: np.ndarray, block: int = BLOCK):
    """H = U D U^T for symmetric positive definite H [k][k]: U unit upper
    block-triangular, D block-diagonal (blocks of `block`), by eliminating
    the blocks from the last one up.  Returns (U, D)."""
    a = np.array(h, dtype=np.float64, copy=True)
    k = a.shape[0]
    nb = k // block
    u = np.eye(k)
    d = np.zeros((k, k))
    for j in range(nb - 1, -1, -1):
        sl = slice(j * block, (j + 1) * block)
        dj = a[sl, sl].copy()
        np.linalg.cholesky(dj)                          # raises unless positive definite
        d[sl, sl] = dj
        if j:
            pre = slice(0, j * block)
            x = np.linalg.solve(dj, a[pre, sl].T).T     # U[pre, block j] = H[pre, j] D_j^-1
            u[pre, sl] = x
            a[pre, pre] = a[pre, pre] - x @ a[pre, sl].T
    return u, d


def ldlq_encode_rotated(w_rot: np.ndarray, h_rot: np.ndarray, block: int = BLOCK, c: float = SCALE_C):
    """Block LDLQ over rotated weights W~ [N][K] with the rotated Hessian
    H~ [K][K]: per block in order the target T_j (feedback summed as stated
    above), its scale, its minimum-squared-error trellis path.  `block` may
    be shortened (a multiple of 4) for tests on tiny blocks.  Returns codes
    u8 [N][K/4], scale bits u16 [N][K/block] and the rounding errors
    eta [N][K] (What - T per block)."""
    w = np.asarray(w_rot, dtype=np.float64)
    n, k = w.shape
    nb, g = k // block, block // 4
    u, _ = block_udu(h_rot, block)
    codes = np.zeros((n, k // 4), dtype=np.uint8)
    scales = np.zeros((n, nb), dtype=np.uint16)
    err = np.zeros((n, k))               # W~ - What of the blocks coded so far
    eta = np.zeros((n, k))
    for j in range(nb):
        sl = slice(j * block, (j + 1) * block)
        acc = np.zeros((n, block))
        for cp in range(j * block):
            acc = acc + err[:, cp:cp + 1] * u[cp, sl][None, :]
        t = w[:, sl] + acc
        sb = block_scale_bits(t, c)
        cj = viterbi_encode(t, sb)
        codes[:, j * g:(j + 1) * g] = cj
        scales[:, j] = sb
        lv = np.array([decode_block_levels(cj[r]) for r in range(n)], dtype=np.float64)
        what = fp16_bits_to_float(sb)[:, None] * lv
        err[:, sl] = w[:, sl] - what
        eta[:, sl] = what - t
    return codes, scales, eta


def encode_matrix_ldlq(w: np.ndarray, sign_bits: np.ndarray, hessian: np.ndarray, c: float = SCALE_C):
    """Offline compression with LDLQ: W [N][K] (fp32 values), the layer
    inputs' proxy Hessian H [K][K] (symmetric positive definite, original
    basis).  Returns codes u8 [N][K/4] and scale bits u16 [N][K/128]."""
    w = np.asarray(w, dtype=np.float32).astype(np.float64)
    wr = rotate(w, sign_bits)
    codes, scales, _ = ldlq_encode_rotated(wr, rotate_hessian(hessian, sign_bits), BLOCK, c)
    return codes, scales


def proxy_loss(w_rot: np.ndarray, what: np.ndarray, h_rot: np.ndarray) -> float:
    """tr(E H~ E^T) with E = What - W~ (fp64)."""
    e = np.asarray(what, dtype=np.float64) - np.asarray(w_rot, dtype=np.float64)
    return float(np.sum((e @ h_rot) * e))


# ------------------------------------------- encoder through a codebook table
def viterbi_encode_table(w_rot: np.ndarray, scale_bits: np.ndarray, table: np.ndarray,
                         rate23: bool = False) -> np.ndarray:
    """Minimum-squared-error path per block through a codebook table, on P8F
    v1's trellis or the rate-2/3 one.  w_rot [nb, 4G] fp64, scale_bits [nb]
    u16, table [8][256][4] int8.  For every group, state p and byte c the
    distortion ((d0^2 + d1^2) + d2^2) + d3^2 with d_j = w_j - s * T[p][c][j];
    for every state and branch u (the byte's branch bits) the first byte of
    least distortion in increasing byte order; then add-compare-select from
    state 0, each next state's predecessors tried in increasing order with
    strict improvement, the first best end state, traceback.  A zero scale
    codes every group as byte 0.  On P8F v1's own table this is
    viterbi_encode, on the rate-2/3 variant's own table viterbi_encode_r23."""
    w = np.asarray(w_rot, dtype=np.float64)
    nb, g = w.shape[0], w.shape[1] // 4
    sv = fp16_bits_to_float(np.asarray(scale_bits, dtype=np.uint16))
    t = np.asarray(table, dtype=np.int8).reshape(8, 256, 4).astype(np.float64)
    nbr = 4 if rate23 else 2
    umask = nbr - 1
    by_u = [np.array([c for c in range(256) if (c & umask) == u], dtype=np.int64) for u in range(nbr)]
    nxt = next_state_r23 if rate23 else next_state
    out = np.zeros((nb, g), dtype=np.uint8)
    for b in range(nb):
        if sv[b] == 0:
            continue
        d = w[b].reshape(g, 1, 1, 4) - sv[b] * t[None, :, :, :]            # [g, 8, 256, 4]
        sq = d * d
        dist = ((sq[..., 0] + sq[..., 1]) + sq[..., 2]) + sq[..., 3]        # [g, 8, 256]
        best_d = np.zeros((g, 8, nbr))
        best_c = np.zeros((g, 8, nbr), dtype=np.int64)
        for u in range(nbr):
            sub = dist[:, :, by_u[u]]
            i = np.argmin(sub, axis=2)                                        # first minimum
            best_d[:, :, u] = np.take_along_axis(sub, i[..., None], axis=2)[..., 0]
            best_c[:, :, u] = by_u[u][i]
        metric = np.full(8, np.inf)
        metric[0] = 0.0
        back = np.zeros((g, 8, 2), dtype=np.int64)
        for step in range(g):
            new = np.full(8, np.inf)
            for p in range(8):                                                # increasing predecessor
                for u in range(nbr):
                    sn = nxt(p, u)
                    tot = metric[p] + best_d[step, p, u]
                    if tot < new[sn]:
                        new[sn] = tot
                        back[step, sn] = (p, best_c[step, p, u])
            metric = new
        st = int(np.argmin(metric))
        for step in range(g - 1, -1, -1):
            out[b, step] = back[step, st, 1]
            st = int(back[step, st, 0])
    return out


def block_distortion_table(w_rot: np.ndarray, codes: np.ndarray, scale_bits: np.ndarray, table: np.ndarray,
                           rate23: bool = False) -> np.ndarray:
    """Squared error per block of codes [nb, G] decoded through the table."""
    w = np.asarray(w_rot, dtype=np.float64)
    g = np.asarray(codes).shape[1]
    pad = (-g) % GROUPS_PER_BLOCK
    c = np.concatenate([np.asarray(codes, dtype=np.uint8), np.zeros((len(codes), pad), np.uint8)], axis=1)
    lv = decode_levels_table(c, table, rate23=rate23).astype(np.float64)[:, :4 * g]
    d = w - fp16_bits_to_float(np.asarray(scale_bits, dtype=np.uint16))[:, None] * lv
    return np.sum(d * d, axis=1)


def encode_matrix_table(w: np.ndarray, sign_bits: np.ndarray, table: np.ndarray, rate23: bool = False,
                        c: float = SCALE_C):
    """Offline compression through a codebook table: rotate, the usual scale
    rule, viterbi_encode_table per block.  Returns codes u8 [N][K/4] and
    scale bits u16 [N][K/128]."""
    w = np.asarray(w, dtype=np.float32).astype(np.float64)
    n, k = w.shape
    wr = rotate(w, sign_bits).reshape(-1, BLOCK)
    sb = block_scale_bits(wr, c)
    codes = viterbi_encode_table(wr, sb, table, rate23)
    return codes.reshape(n, k // 4), sb.reshape(n, k // BLOCK)
