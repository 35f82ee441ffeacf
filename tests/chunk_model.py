"""Float64 NumPy model of the GPU chunked algorithm (CPU test aid, not the oracle).

It mirrors the decomposition the HIP kernels use, so the algebra can be
checked against the oracle before and independently of any GPU run:

  * the token axis is cut, in original token order, into segments of L tokens
    and each segment into sub-chunks of c = 64 tokens (the last of each may be
    ragged); a scan direction visits segments, sub-chunks and tokens in its own
    order (ascending for the forward scan, descending for the reversed one);
  * sub-chunk form, with G the inclusive within-sub-chunk cumsum of the
    log-gates in scan order and E_ij = exp(G_i - G_j) (only i >= j is used):
        A  = strict_lower(diag(beta) K K^T * E)
        Tm = (I + A)^-1      (16x16 diagonal blocks by substitution, then
                              off-diagonal blocks level by level)
        R  = V - diag(exp(G)) K H          (values minus the decayed prediction)
        V' = Tm diag(beta) R
        O  = diag(exp(G)) Q H + (tril(Q K^T) * E) V'
        H <- exp(G_n) H + (diag(exp(G_n - G)) K)^T V'
    (equal to the WY/UT form V' = U - W H with W = Tm diag(beta exp(G)) K and
    U = Tm diag(beta) V, which `wy` keeps for the tests);
  * segment map (phase 1): the same chain run on X = [P | Q] from [I | 0] with
    values [0 | V] gives H_end = P H_start + Q;
  * segment chain (phase 2): H_{s+1} = P_s H_s + Q_s;
  * output pass (phase 3): each segment re-run from its true start state.
"""
import numpy as np

C = 64


def subchunks(T, L):
    """[(segment, [(start, stop) of its sub-chunks])] in original token order."""
    segs = []
    for s0 in range(0, T, L):
        s1 = min(s0 + L, T)
        segs.append([(a, min(a + C, s1)) for a in range(s0, s1, C)])
    return segs


def wy(K, V, g, beta):
    """Sub-chunk WY/UT quantities for tokens already in scan order."""
    n = len(g)
    G = np.cumsum(g)
    E = np.exp(np.tril(G[:, None] - G[None, :]))
    A = np.tril((beta[:, None] * (K @ K.T)) * E, -1)
    Tm = np.linalg.inv(np.eye(n) + A)
    W = Tm @ ((beta * np.exp(G))[:, None] * K)
    U = Tm @ (beta[:, None] * V)
    return G, E, W, U


def blocked_inverse(A, blk=16):
    """(I + A)^-1 for strictly lower A, n a multiple of blk: each diagonal block
    by row-wise substitution T_ii (I + A_ii) = I, then the off-diagonal blocks
    T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj, level i - j = 1, 2, ..."""
    n = A.shape[0]
    nb = n // blk
    T = np.zeros_like(A)
    for b in range(nb):
        Ab = A[b * blk:(b + 1) * blk, b * blk:(b + 1) * blk]
        for i in range(blk):
            s = np.zeros(blk)
            s[i] = 1.0
            for k in range(blk - 1, -1, -1):
                s[:k] -= s[k] * Ab[k, :k]
            T[b * blk + i, b * blk:(b + 1) * blk] = s
    S = lambda i: slice(i * blk, (i + 1) * blk)
    for lev in range(1, nb):
        for j in range(nb - lev):
            i = j + lev
            M = sum(A[S(i), S(k)] @ T[S(k), S(j)] for k in range(j, i))
            T[S(i), S(j)] = -T[S(i), S(i)] @ M
    return T


def chunk_step(H, Q, K, V, g, beta):
    """One sub-chunk from state H: returns (outputs, new state)."""
    n = len(g)
    G = np.cumsum(g)
    E = np.exp(np.tril(G[:, None] - G[None, :]))
    A = np.tril((beta[:, None] * (K @ K.T)) * E, -1)
    pad = (-n) % 16
    Ap = np.pad(A, ((0, pad), (0, pad)))
    Tm = blocked_inverse(Ap)[:n, :n]
    R = V - np.exp(G)[:, None] * (K @ H)
    Vn = Tm @ (beta[:, None] * R)
    O = np.exp(G)[:, None] * (Q @ H) + (np.tril(Q @ K.T) * E) @ Vn
    Hn = np.exp(G[-1]) * H + (np.exp(G[-1] - G)[:, None] * K).T @ Vn
    return O, Hn


def segment_map(K, V, g, beta, pieces):
    """Phase 1: P, Q of one segment (pieces in scan order, local indices)."""
    dk, dv = K.shape[1], V.shape[1]
    X = np.concatenate([np.eye(dk), np.zeros((dk, dv))], axis=1)
    for idx in pieces:
        Va = np.concatenate([np.zeros((len(idx), dk)), V[idx]], axis=1)
        _, X = chunk_step(X, np.zeros((len(idx), dk)), K[idx], Va, g[idx], beta[idx])
    return X[:, :dk], X[:, dk:]


def scan_one(q, k, v, g, beta, h0, L, reverse):
    """One direction for one (batch, head): q,k [T,dk], v [T,dv], g,beta [T]."""
    T = len(g)
    segs = subchunks(T, L)
    order = list(range(len(segs)))
    if reverse:
        order = order[::-1]

    def pieces(seg):
        ps = [np.arange(a, b) for a, b in segs[seg]]
        return [p[::-1] for p in ps[::-1]] if reverse else ps

    # phase 1: maps of every segment in scan order
    maps = [segment_map(k, v, g, beta, pieces(s)) for s in order]
    # phase 2: start states
    H = h0.copy()
    starts = []
    for P, Qm in maps:
        starts.append(H)
        H = P @ H + Qm
    # phase 3: outputs
    o = np.zeros((T, v.shape[1]))
    for H, s in zip(starts, order):
        for idx in pieces(s):
            O, H = chunk_step(H, q[idx], k[idx], v[idx], g[idx], beta[idx])
            o[idx] = O
    return o, H


def forward(direction, q, k, v, log_gate, beta, h0=None, key_scale=1.0, L=256):
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64) * key_scale
    v = np.asarray(v, np.float64)
    g = np.asarray(log_gate, np.float64)
    b = np.asarray(beta, np.float64)
    B, T, Hh, dk = q.shape
    dv = v.shape[-1]
    h0 = np.zeros((B, Hh, dk, dv)) if h0 is None else np.asarray(h0, np.float64)
    o = np.zeros((B, T, Hh, dv))
    hT = np.zeros((B, Hh, dk, dv))
    for bi in range(B):
        for h in range(Hh):
            a = (q[bi, :, h], k[bi, :, h], v[bi, :, h], g[bi, :, h], b[bi, :, h])
            if direction == "fwd":
                o[bi, :, h], hT[bi, h] = scan_one(*a, h0[bi, h], L, False)
            elif direction == "bwd":
                o[bi, :, h], hT[bi, h] = scan_one(*a, h0[bi, h], L, True)
            else:
                of, hT[bi, h] = scan_one(*a, h0[bi, h], L, False)
                ob, _ = scan_one(*a, np.zeros((dk, dv)), L, True)
                o[bi, :, h] = of + ob
    return o, hT
