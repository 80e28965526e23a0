"""Dense NumPy brute force used to pin the CPU oracle (test code only).

Written independently of oracle.c: it decodes the documented code layout with array
reshapes instead of per-element index arithmetic, dequantises whole matrices, and
evaluates EVERY expert on EVERY row with dense float64 matrix products, masking to the
chosen top-k afterwards (the check the layer's definition asks for: dense evaluation
of all experts, masked to the routing). It also holds the inverse of the layout (a
packer) so tests can place known codes and read them back through the oracle.
"""
import numpy as np


def group_width(bits):
    return 512 // bits


def unpack_codes(codes, rows, cols, bits):
    """Dense integer codes [rows, cols] of one matrix from its packed bytes."""
    G = group_width(bits)
    T, NG, nb = rows // 16, cols // G, G // 32
    lanes = np.asarray(codes, np.uint8).reshape(T, NG, 64, 16)
    bitsarr = np.unpackbits(lanes, axis=-1, bitorder="little")          # [T,NG,64,128]
    fields = bitsarr.reshape(T, NG, 64, 128 // bits, bits)
    vals = (fields.astype(np.int64) << np.arange(bits)).sum(-1)         # [T,NG,64,8*nb]
    if bits == 8:
        vals = np.where(vals >= 128, vals - 256, vals)
    # lane = 16*j + n_in ; field = 8*beta + i
    vals = vals.reshape(T, NG, 4, 16, nb, 8)                            # t g j n beta i
    vals = vals.transpose(0, 3, 1, 4, 2, 5)                             # t n g beta j i
    return vals.reshape(rows, cols)


def pack_codes(dense, bits):
    """Inverse of unpack_codes: packed bytes of a dense integer code matrix."""
    dense = np.asarray(dense, np.int64)
    rows, cols = dense.shape
    G = group_width(bits)
    T, NG, nb = rows // 16, cols // G, G // 32
    v = dense.reshape(T, 16, NG, nb, 4, 8).transpose(0, 2, 4, 1, 3, 5)  # t g j n beta i
    v = v.reshape(T, NG, 64, 128 // bits) & ((1 << bits) - 1)
    b = ((v[..., None] >> np.arange(bits)) & 1).astype(np.uint8)
    b = b.reshape(T, NG, 64, 128)
    return np.packbits(b, axis=-1, bitorder="little").reshape(-1)


def unpack_meta(meta, rows, cols, bits):
    """(scale, min) float64 arrays [rows, cols/32] of one matrix."""
    G = group_width(bits)
    T, NG, nb = rows // 16, cols // G, G // 32
    m = np.asarray(meta).reshape(T, NG, 16, nb).transpose(0, 2, 1, 3).reshape(rows, cols // 32)
    if bits == 8:
        return m.astype(np.uint16).view(np.float16).astype(np.float64), np.zeros(m.shape)
    s = (m & 0xFFFF).astype(np.uint16).view(np.float16).astype(np.float64)
    mn = (m >> 16).astype(np.uint16).view(np.float16).astype(np.float64)
    return s, mn


def pack_meta(scale, mn, bits):
    """Inverse of unpack_meta (binary16 inputs given as float arrays [rows, cols/32])."""
    rows, nblk = scale.shape
    G = group_width(bits)
    nb = G // 32
    T, NG = rows // 16, nblk // nb
    s = np.asarray(scale, np.float16).view(np.uint16)
    if bits == 8:
        out = s
    else:
        out = s.astype(np.uint32) | (np.asarray(mn, np.float16).view(np.uint16).astype(np.uint32) << 16)
    return out.reshape(T, 16, NG, nb).transpose(0, 2, 1, 3).reshape(-1)


def dequant(codes, meta, rows, cols, bits):
    q = unpack_codes(codes, rows, cols, bits).astype(np.float64)
    s, mn = unpack_meta(meta, rows, cols, bits)
    return q * np.repeat(s, 32, axis=1) + np.repeat(mn, 32, axis=1)


def act(x):
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def silu(z):
    from scipy.special import expit
    return z * expit(z)


def dense_ffn(Wg, Wu, Wd, X):
    """SwiGLU FFN of all rows X [R, H] with dense float64 weights."""
    return (silu(X @ Wg.T) * (X @ Wu.T)) @ Wd.T


def route_bruteforce(X, G, bias, k, renorm):
    logits = X @ np.asarray(G, np.float64).T
    if bias is not None:
        logits = logits + np.asarray(bias, np.float64)
    from scipy.special import softmax
    probs = softmax(logits, axis=1)
    R, E = logits.shape
    idx = np.empty((R, k), np.int64)
    for r in range(R):
        order = np.lexsort((np.arange(E), -logits[r]))  # by -logit, then index
        idx[r] = order[:k]
    w = np.take_along_axis(probs, idx, axis=1)
    if renorm:
        w = w / w.sum(axis=1, keepdims=True)
    return logits, probs, idx, w


def layer_dense(x, layer, cfg, renorm=False, residual=False):
    """Brute force of a whole MoE layer: every expert on every row, masked to top-k."""
    X = act(x)
    R, H = X.shape
    E, F, b = cfg.experts, cfg.ffn, cfg.bits
    _, _, idx, w = route_bruteforce(X, layer.gate_w, layer.bias, cfg.top_k, renorm)
    mask = np.zeros((R, E))
    for r in range(R):
        for j in range(cfg.top_k):
            mask[r, idx[r, j]] = w[r, j]
    out = np.zeros((R, H))
    for e in range(E):
        Y = dense_ffn(dequant(layer.gate[0][e], layer.gate[1][e], F, H, b),
                      dequant(layer.up[0][e], layer.up[1][e], F, H, b),
                      dequant(layer.down[0][e], layer.down[1][e], H, F, b), X)
        out += mask[:, e:e + 1] * Y
    out += dense_ffn(dequant(layer.sh_gate[0][0], layer.sh_gate[1][0], F, H, b),
                     dequant(layer.sh_up[0][0], layer.sh_up[1][0], F, H, b),
                     dequant(layer.sh_down[0][0], layer.sh_down[1][0], H, F, b), X)
    if residual:
        out += X
    return out, idx, w
