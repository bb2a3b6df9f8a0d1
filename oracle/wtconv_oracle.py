"""Plain fp64 CPU oracle for the WTConv operator, forward and backward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code, table or helper with the HIP
library and imports nothing from it.

What is computed (source: "Fast and Memory-Efficient Wavelet Convolutions via
I/O-Aware Reformulation", arXiv 2608.10805, Abstract -- WTConv is a
multi-level Haar wavelet decomposition, a depthwise convolution with learned
per-channel scales on every level's subbands, a synthesis back to full
resolution, and a base depthwise convolution).  The oracle implements that
definition literally, level by level, as the unfused cascade, in float64:

  LL_0 = x
  for i = 1..L:   pad LL_{i-1} right/bottom to even size with zeros,
                  (S_i^0, S_i^1, S_i^2, S_i^3) = orthonormal 2x2 Haar analysis
                  (factor 1/2), LL_i = S_i^0
  Y_i = s_i * dwconv_k(S_i, W_i)          over the 4C subband-channels 4c+u,
                                          zero padding k//2, stride 1
  Z_{L+1} = 0
  Z_i = inverse Haar(Y_i^0 + Z_{i+1}, Y_i^1, Y_i^2, Y_i^3), cropped to the
        size of LL_{i-1}
  out = s0 * dwconv_k(x, W0) + b0 + Z_1

Readings taken where the pages are silent (each one is a plain reading):
  * subband index u = 2*u_y + u_x; with a=(0,0), b=(0,1), c=(1,0), d=(1,1)
    of a 2x2 block: LL=(a+b+c+d)/2, u=1 (high-pass along W)=(a-b+c-d)/2,
    u=2 (high-pass along H)=(a+b-c-d)/2, u=3=(a-b-c+d)/2.  This 4x4 matrix is
    symmetric and orthogonal, so it is its own inverse (the textbook Haar
    facts: orthogonal transform, inverse = transpose -- SETAREH article,
    paragraph on the Haar wavelet transform).
  * the scale s_i has one entry per subband-channel (shape [L, 4C]), like
    the leading dimension of W_i;
  * the bias b0 sits outside s0;
  * "dwconv" is cross-correlation (W * X)[p] = sum_d W[d + r] X[p + d];
  * the raw (unconvolved) LL band feeds the next level; every level's
    convolved LL band enters the synthesis.

The backward pass is the hand-written adjoint of each forward step, taken in
reverse order (crop <-> zero-pad, synthesis <-> analysis because the Haar
matrix is symmetric orthogonal, correlation <-> 180-degree-rotated
correlation).  Scale gradients are computed directly as sum(dY * conv),
not through any weight-folding identity.

Layouts (all float64 on output):
  x, g   [B, C, H, W]
  w0     [C, k, k]      s0, b0 [C]
  wl     [L, 4C, k, k]  sl     [L, 4C]     (subband-channel index 4c+u)
"""

import numpy as np

__all__ = [
    "haar2_analysis",
    "haar2_synthesis",
    "dwconv",
    "corr",
    "forward",
    "backward",
]


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def _pad_even(X):
    """Zero-pad the last two axes on the bottom/right up to even length."""
    h, w = X.shape[-2:]
    ph, pw = h % 2, w % 2
    if ph == 0 and pw == 0:
        return X
    pad = [(0, 0)] * (X.ndim - 2) + [(0, ph), (0, pw)]
    return np.pad(X, pad)


def haar2_analysis(X):
    """One level of the orthonormal 2x2 Haar analysis.

    X [..., h, w] -> bands [..., 4, ceil(h/2), ceil(w/2)] with the band index
    u = 2*u_y + u_x (u_x: high-pass along W, u_y: high-pass along H).
    """
    Xp = _pad_even(X)
    a = Xp[..., 0::2, 0::2]
    b = Xp[..., 0::2, 1::2]
    c = Xp[..., 1::2, 0::2]
    d = Xp[..., 1::2, 1::2]
    ll = 0.5 * (a + b + c + d)
    hx = 0.5 * (a - b + c - d)
    hy = 0.5 * (a + b - c - d)
    hh = 0.5 * (a - b - c + d)
    return np.stack([ll, hx, hy, hh], axis=-3)


def haar2_synthesis(T, h, w):
    """Inverse of :func:`haar2_analysis`: bands [..., 4, h2, w2] -> [..., h, w].

    The 2x2 Haar matrix is symmetric and orthogonal, so the inverse applies
    the same matrix; the result is cropped to (h, w).
    """
    t0, t1, t2, t3 = T[..., 0, :, :], T[..., 1, :, :], T[..., 2, :, :], T[..., 3, :, :]
    h2, w2 = t0.shape[-2:]
    out = np.zeros(T.shape[:-3] + (2 * h2, 2 * w2), dtype=np.float64)
    out[..., 0::2, 0::2] = 0.5 * (t0 + t1 + t2 + t3)
    out[..., 0::2, 1::2] = 0.5 * (t0 - t1 + t2 - t3)
    out[..., 1::2, 0::2] = 0.5 * (t0 + t1 - t2 - t3)
    out[..., 1::2, 1::2] = 0.5 * (t0 - t1 - t2 + t3)
    return out[..., :h, :w]


def dwconv(X, Wk):
    """Depthwise cross-correlation with zero padding k//2 (same-size output).

    X [B, C, h, w], Wk [C, k, k]:  out[b,c,p] = sum_d Wk[c, d+r] X[b,c,p+d].
    Computed as k*k shifted-slice accumulations.
    """
    X = _f64(X)
    Wk = _f64(Wk)
    k = Wk.shape[-1]
    r = k // 2
    h, w = X.shape[-2:]
    Xp = np.pad(X, [(0, 0), (0, 0), (r, r), (r, r)])
    out = np.zeros_like(X)
    for ky in range(k):
        for kx in range(k):
            out += Wk[None, :, ky, kx, None, None] * Xp[:, :, ky:ky + h, kx:kx + w]
    return out


def corr(A, X, k):
    """Weight-gradient correlation summed over batch and space.

    A, X [B, C, h, w] -> [C, k, k]:  out[c, d+r] = sum_{b,p} A[b,c,p] X[b,c,p+d],
    X taken as zero outside its grid.
    """
    A = _f64(A)
    X = _f64(X)
    r = k // 2
    h, w = X.shape[-2:]
    Xp = np.pad(X, [(0, 0), (0, 0), (r, r), (r, r)])
    out = np.zeros((X.shape[1], k, k), dtype=np.float64)
    for ky in range(k):
        for kx in range(k):
            out[:, ky, kx] = np.einsum("bchw,bchw->c", A, Xp[:, :, ky:ky + h, kx:kx + w])
    return out


def _rot180(Wk):
    return Wk[..., ::-1, ::-1]


def _analysis_cascade(x, L):
    """Bands S_i [B, C, 4, h_i, w_i] for i = 1..L and the LL sizes before each level."""
    LL = x
    S, sizes = [], []
    for _ in range(L):
        sizes.append(LL.shape[-2:])
        bands = haar2_analysis(LL)
        S.append(bands)
        LL = bands[:, :, 0]
    return S, sizes


def _check(x, w0, s0, b0, wl, sl, L):
    B, C, H, W = x.shape
    k = w0.shape[-1]
    assert w0.shape == (C, k, k) and k % 2 == 1
    assert s0.shape == (C,) and (b0 is None or b0.shape == (C,))
    if L > 0:
        assert wl.shape[0] >= L and wl.shape[1:] == (4 * C, k, k)
        assert sl.shape[0] >= L and sl.shape[1] == 4 * C
    return B, C, k


def _forward_chunk(x, w0, s0, b0, wl, sl, L):
    B, C, k = _check(x, w0, s0, b0, wl, sl, L)
    S, sizes = _analysis_cascade(x, L)
    Z = None
    for i in range(L, 0, -1):
        Si = S[i - 1]
        h, w = Si.shape[-2:]
        Yi = sl[i - 1][None, :, None, None] * dwconv(Si.reshape(B, 4 * C, h, w), wl[i - 1])
        T = Yi.reshape(B, C, 4, h, w).copy()
        if Z is not None:
            T[:, :, 0] += Z
        Z = haar2_synthesis(T, *sizes[i - 1])
    out = s0[None, :, None, None] * dwconv(x, w0)
    if b0 is not None:
        out = out + b0[None, :, None, None]
    if Z is not None:
        out = out + Z
    return out


def forward(x, w0, s0, b0, wl, sl, L, batch_chunk=None):
    """WTConv forward in float64.  Returns out [B, C, H, W]."""
    x, w0, s0, b0, wl, sl = map(_f64, (x, w0, s0, b0, wl, sl))
    B = x.shape[0]
    bc = B if batch_chunk is None else max(1, int(batch_chunk))
    parts = [_forward_chunk(x[i:i + bc], w0, s0, b0, wl, sl, L) for i in range(0, B, bc)]
    return np.concatenate(parts, axis=0)


def _backward_chunk(x, g, w0, s0, b0, wl, sl, L):
    B, C, k = _check(x, w0, s0, b0, wl, sl, L)
    S, sizes = _analysis_cascade(x, L)

    # Adjoint of the synthesis cascade: dZ_1 = g; dT_i = analysis(pad(dZ_i)),
    # dY_i = dT_i, dZ_{i+1} = dT_i^0.
    dY = []
    dZ = g
    for _ in range(L):
        dT = haar2_analysis(dZ)
        dY.append(dT)
        dZ = dT[:, :, 0]

    dwl = np.zeros((L, 4 * C, k, k)) if L > 0 else None
    dsl = np.zeros((L, 4 * C)) if L > 0 else None
    dS = []
    for i in range(1, L + 1):
        Si = S[i - 1]
        h, w = Si.shape[-2:]
        Sf = Si.reshape(B, 4 * C, h, w)
        dYf = dY[i - 1].reshape(B, 4 * C, h, w)
        V = dwconv(Sf, wl[i - 1])  # unscaled conv output
        dwl[i - 1] = sl[i - 1][:, None, None] * corr(dYf, Sf, k)
        dsl[i - 1] = np.einsum("bchw,bchw->c", dYf, V)
        dSf = sl[i - 1][None, :, None, None] * dwconv(dYf, _rot180(wl[i - 1]))
        dS.append(dSf.reshape(B, C, 4, h, w))

    # Adjoint of the analysis cascade, deepest level first.
    dLL = None
    for i in range(L, 0, -1):
        T = dS[i - 1].copy()
        if dLL is not None:
            T[:, :, 0] += dLL
        dLL = haar2_synthesis(T, *sizes[i - 1])

    dx = s0[None, :, None, None] * dwconv(g, _rot180(w0))
    if dLL is not None:
        dx = dx + dLL
    dw0 = s0[:, None, None] * corr(g, x, k)
    ds0 = np.einsum("bchw,bchw->c", g, dwconv(x, w0))
    db0 = g.sum(axis=(0, 2, 3))
    return dict(dx=dx, dw0=dw0, ds0=ds0, db0=db0, dwl=dwl, dsl=dsl)


def backward(x, g, w0, s0, b0, wl, sl, L, batch_chunk=None):
    """Gradients of <g, forward(...)> in float64.

    Returns a dict with dx [B,C,H,W], dw0 [C,k,k], ds0 [C], db0 [C],
    dwl [L,4C,k,k] and dsl [L,4C] (the last two are None when L == 0).
    Parameter gradients are with respect to the unscaled weights W.
    """
    x, g, w0, s0, b0, wl, sl = map(_f64, (x, g, w0, s0, b0, wl, sl))
    B = x.shape[0]
    bc = B if batch_chunk is None else max(1, int(batch_chunk))
    total = None
    dxs = []
    for i in range(0, B, bc):
        part = _backward_chunk(x[i:i + bc], g[i:i + bc], w0, s0, b0, wl, sl, L)
        dxs.append(part.pop("dx"))
        if total is None:
            total = part
        else:
            for key, val in part.items():
                if val is not None:
                    total[key] = total[key] + val
    total["dx"] = np.concatenate(dxs, axis=0)
    return total
