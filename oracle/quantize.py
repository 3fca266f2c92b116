"""Mixed-width group quantisation and the packed cache layout.

Test infrastructure only (see the package docstring).

RDKV summary, §2.2: each retained unit is stored at its allocated width, 2/4/8-bit codes or
16 bits; width 0 stores nothing.  §2.3: the packed store groups rows by width so every
width has a uniform dequantisation path.  The pages fix only the width set; the group size
(32), the asymmetric min-max rule, round-half-even and the float32 scale/zero are the
workload settings.  The byte layout below is this library's own format (parity unpinned: a
convention, not something the pages define).

Quantiser, per group x of up to 32 bf16 values at width b in {2,4,8}:
    z = min(x) (exact in float32),
    s = RN32( RN64( RN64(max(x) - z) / (2^b - 1) ) ),
    code = clamp( round_half_even( RN64((x - z) / s) ), 0, 2^b - 1 ),  all codes 0 if s == 0.
Word packing: element e of a group occupies bits [e*b, e*b + b) of the group's little-endian
stream of 32-bit words, so a 32-element group at width b is exactly b words; at b = 16 the
stream is the raw bf16 bits; a short (tail) group is padded with code 0.

Grouping axes (a reading; the pages are silent): V groups run along the d channels of one
token; K groups run along the retained tokens of one channel, in ascending token order.
"""

import numpy as np

from .common import as_f64

WIDTHS = (2, 4, 8, 16)           # zone z <-> WIDTHS[z]
HDR_GLOBAL = 16
HDR_PER_HEAD = 24
VLOC_SHIFT = 29


def quantize_group(x, b):
    """Quantise one or many groups (rows of ``x``, float64 bf16 values) at width b in {2,4,8}.

    Returns (codes int64 same shape, scale float32 [rows], zero float32 [rows]).
    """
    X = np.atleast_2d(np.asarray(x, dtype=np.float64))
    z = X.min(axis=1)
    mx = X.max(axis=1)
    s32 = ((mx - z) / float(2 ** b - 1)).astype(np.float32)
    s = s32.astype(np.float64)
    codes = np.zeros(X.shape, dtype=np.int64)
    nz = s > 0
    if nz.any():
        v = (X[nz] - z[nz, None]) / s[nz, None]
        codes[nz] = np.clip(np.rint(v), 0, 2 ** b - 1).astype(np.int64)
    return codes, s32, z.astype(np.float32)


def pack_group_words(codes, b):
    """Pack rows of up to 32 codes (pad with 0) into b uint32 words each, LSB first."""
    C = np.atleast_2d(np.asarray(codes, dtype=np.uint64))
    n, m = C.shape
    words = np.zeros((n, b), dtype=np.uint64)
    for e in range(m):
        bit = e * b
        words[:, bit // 32] |= (C[:, e] & np.uint64((1 << b) - 1)) << np.uint64(bit % 32)
    return words.astype(np.uint32)


def _check_widths(a, what):
    a = np.asarray(a)
    bad = ~np.isin(a, (0, 2, 4, 8, 16))
    if bad.any():
        raise ValueError(f"{what} holds a width outside {{0,2,4,8,16}}")


def pack_cache(k, v, bits_v, bits_k, group_size=32):
    """Build the packed cache of one layer (all KV heads).

    Inputs: K, V bf16 bits [H_kv][N][d]; bits_v uint8 [H_kv][N]; bits_k uint8 [H_kv][d].
    A token is retained iff bits_v > 0.  Returns a dict of numpy arrays, each trimmed to the
    length actually used:
      header  int64   [HDR_GLOBAL + H_kv*HDR_PER_HEAD]
      v_idx   int32   token ids, per (head, zone) in zone order 2,4,8,16, ascending
      v_words uint32  per listed token: d/32 groups x b words
      v_par   float32 [pairs][2] (scale, zero) per listed token per group, zones 2/4/8 only
      k_keep  int32   retained token ids per head, ascending
      k_vloc  int32   per retained token: zone << 29 | position within its V zone
      k_words uint32  per head, per group j of 32 retained tokens, per channel c (ascending)
                      with bits_k[c] > 0: bits_k[c] words
      k_par   float32 [pairs][2] per (group j, channel c with bits_k[c] in {2,4,8})
      k_width uint8   [H_kv][d] copy of bits_k
    """
    if group_size != 32:
        raise ValueError("group size 32 only")
    K = np.asarray(k, dtype=np.uint16)
    V = np.asarray(v, dtype=np.uint16)
    bv = np.asarray(bits_v, dtype=np.uint8)
    bk = np.asarray(bits_k, dtype=np.uint8)
    _check_widths(bv, "bits_v")
    _check_widths(bk, "bits_k")
    hkv, n, d = K.shape
    if d % 32:
        raise ValueError("head_dim must be a multiple of 32")
    gpr = d // 32                                     # V groups per token
    hdr = np.zeros(HDR_GLOBAL + hkv * HDR_PER_HEAD, dtype=np.int64)
    hdr[0:4] = (hkv, d, n, group_size)

    v_idx, v_words, v_par = [], [], []
    k_keep, k_vloc, k_words, k_par = [], [], [], []
    o_vi = o_vw = o_vp = o_kk = o_kw = o_kp = 0
    for g in range(hkv):
        base = HDR_GLOBAL + g * HDR_PER_HEAD
        kept = np.nonzero(bv[g] > 0)[0]
        R = kept.size
        zone_of = np.full(n, -1, dtype=np.int64)
        pos_of = np.full(n, -1, dtype=np.int64)
        for z, b in enumerate(WIDTHS):
            toks = np.nonzero(bv[g] == b)[0]
            nv = toks.size
            hdr[base + z] = nv
            hdr[base + 5 + z] = o_vi
            hdr[base + 9 + z] = o_vw
            hdr[base + 13 + z] = o_vp
            zone_of[toks] = z
            pos_of[toks] = np.arange(nv)
            v_idx.append(toks.astype(np.int32))
            if nv:
                if b == 16:
                    raw = V[g][toks].reshape(nv * gpr, 32).astype(np.uint64)
                    w = pack_group_words(raw, 16)
                else:
                    x = as_f64(V[g][toks]).reshape(nv * gpr, 32)
                    codes, s, zz = quantize_group(x, b)
                    w = pack_group_words(codes, b)
                    v_par.append(np.stack([s, zz], axis=1))
                v_words.append(w.reshape(-1))
            o_vi += nv
            o_vw += nv * gpr * b
            o_vp += nv * gpr if b != 16 else 0
        hdr[base + 4] = R
        hdr[base + 17] = o_kk
        hdr[base + 18] = o_kw
        hdr[base + 19] = o_kp
        chans = [c for c in range(d) if bk[g, c] > 0]
        qchans = [c for c in chans if bk[g, c] != 16]
        wk = int(sum(int(bk[g, c]) for c in chans))
        ngroups = (R + 31) // 32
        hdr[base + 20] = wk
        hdr[base + 21] = len(qchans)
        hdr[base + 22] = ngroups
        k_keep.append(kept.astype(np.int32))
        k_vloc.append(((zone_of[kept] << VLOC_SHIFT) | pos_of[kept]).astype(np.int32))
        # group-major: row j holds, for each kept channel in ascending order, its b words
        kw = np.zeros((ngroups, wk), dtype=np.uint32)
        kp = np.zeros((ngroups, len(qchans), 2), dtype=np.float32)
        woff = 0
        qoff = 0
        for c in chans:
            b = int(bk[g, c])
            col = K[g][kept, c]                                   # retained tokens, ascending
            nfull = R // 32
            for j0, j1, rows in ((0, nfull, col[:32 * nfull].reshape(nfull, 32)),   # full groups
                                 (nfull, ngroups, col[32 * nfull:][None, :])):        # short tail
                if j1 <= j0:
                    continue
                if b == 16:
                    kw[j0:j1, woff:woff + b] = pack_group_words(rows.astype(np.uint64), 16)
                else:
                    codes, s, zz = quantize_group(as_f64(rows), b)
                    kw[j0:j1, woff:woff + b] = pack_group_words(codes, b)
                    kp[j0:j1, qoff, 0] = s
                    kp[j0:j1, qoff, 1] = zz
            woff += b
            if b != 16:
                qoff += 1
        k_words.append(kw.reshape(-1))
        k_par.append(kp.reshape(-1, 2))
        o_kk += R
        o_kw += ngroups * wk
        o_kp += ngroups * len(qchans)
    hdr[4:10] = (o_vi, o_vw, o_vp, o_kk, o_kw, o_kp)

    def cat(parts, dtype, shape_tail=()):
        parts = [p for p in parts if p.size]
        if not parts:
            return np.zeros((0,) + shape_tail, dtype=dtype)
        return np.concatenate(parts).astype(dtype)

    return {
        "header": hdr,
        "v_idx": cat(v_idx, np.int32),
        "v_words": cat(v_words, np.uint32),
        "v_par": cat(v_par, np.float32, (2,)),
        "k_keep": cat(k_keep, np.int32),
        "k_vloc": cat(k_vloc, np.int32),
        "k_words": cat(k_words, np.uint32),
        "k_par": cat(k_par, np.float32, (2,)),
        "k_width": bk.copy(),
    }
