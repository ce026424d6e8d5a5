"""Oracle paged attention in float64 (test infrastructure only).

The method computes exact attention: the pages say the block-table lookup is
transparent to the model and leaves the arithmetic that of ordinary attention
(DataWhale notes section 3; vLLM course ch. 4, "key point" after the
pseudocode).  So the oracle is the plain definition, written out:

1. gather each sequence's K and V from its blocks (``cache.gather``);
2. for each head h and query row r, scores s_j = scale * <q_r, k_j> over the
   keys row r may see;
3. p = exp(s - max s), out_r = sum_j p_j v_j / sum_j p_j.

(PagedAttention blog article, section 3.2.2 forward pass: gather, Q K^T
divided by sqrt(head_dim), causal mask, softmax, weighted sum of V, output
zero-initialised.)  Readings of that listing:

* scores are per head, Q_h K_h^T (the listing's matmul shapes do not line up);
* one softmax over all visible keys (the course pseudocode puts it inside the
  token loop);
* ``scale`` is an explicit argument; the configurations use 1/sqrt(head_dim);
* the causal mask is aligned bottom-right: with S query rows at the end of a
  sequence of L tokens, row r sees keys 0 .. L - S + r.  A decode step
  (S = 1) therefore sees every cached token; with no earlier context (S = L)
  this is the usual lower-triangular mask;
* a sequence of length 0 yields zeros;
* fp8 storage is dequantised as code value times the block's scale.
"""
import numpy as np

from . import cache as C


def attend(q, K, V, scale, visible):
    """Softmax attention for query rows q [S, D] over K, V [L, D], float64.

    visible[r] = number of leading keys row r may see (>= 0).
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    out = np.zeros((q.shape[0], V.shape[1]), dtype=np.float64)
    for r in range(q.shape[0]):
        n = int(visible[r])
        if n == 0:
            continue
        s = scale * (K[:n] @ q[r])
        p = np.exp(s - s.max())
        out[r] = (p @ V[:n]) / p.sum()
    return out


def gathered_kv(k_bits, v_bits, kv_dtype, table, length, block_size, k_scale=None, v_scale=None):
    """Float64 K, V of one sequence: [L, H, D] each, dequantised for fp8."""
    K = C.to_float64(C.gather(k_bits, table, length, block_size), kv_dtype)
    V = C.to_float64(C.gather(v_bits, table, length, block_size), kv_dtype)
    if kv_dtype == C.FP8:
        K = K * C.gather_scales(k_scale, table, length, block_size)[:, :, None]
        V = V * C.gather_scales(v_scale, table, length, block_size)[:, :, None]
    return K, V


def decode_one(q_hd, k_bits, v_bits, kv_dtype, table, length, block_size, scale, head,
               k_scale=None, v_scale=None):
    """One (sequence, head) of a decode step: q_hd [D] float64 -> out [D]."""
    K, V = gathered_kv(k_bits, v_bits, kv_dtype, table, length, block_size, k_scale, v_scale)
    return attend(np.asarray(q_hd)[None, :], K[:, head, :], V[:, head, :], scale, [length])[0]


def decode(q, k_bits, v_bits, kv_dtype, tables, lens, block_size, scale,
           k_scale=None, v_scale=None):
    """Decode step: q [B, H, D] float64 (one token per sequence) -> out [B, H, D].

    The query is the sequence's last position, so it sees all L_i keys.
    """
    q = np.asarray(q, dtype=np.float64)
    B, H, D = q.shape
    out = np.zeros((B, H, D), dtype=np.float64)
    for i in range(B):
        K, V = gathered_kv(k_bits, v_bits, kv_dtype, tables[i], int(lens[i]), block_size,
                           k_scale, v_scale)
        for h in range(H):
            out[i, h] = attend(q[i, h][None, :], K[:, h, :], V[:, h, :], scale, [int(lens[i])])[0]
    return out


def chunk_visible(length, num_q):
    """Keys visible to each of the num_q rows at the end of a length-L sequence."""
    return [length - num_q + r + 1 for r in range(num_q)]


def prefill_chunk(q, query_start_loc, k_bits, v_bits, kv_dtype, tables, lens, block_size,
                  scale, heads=None, k_scale=None, v_scale=None):
    """Causal chunk attention: q packed [T, H, D] float64 -> out [T, H, D].

    Sequence i owns rows query_start_loc[i] .. query_start_loc[i+1]-1 of q;
    they are its last S_i positions (lens[i] counts the chunk too).
    ``heads`` restricts the work to a subset of heads (others stay zero).
    """
    q = np.asarray(q, dtype=np.float64)
    T, H, D = q.shape
    out = np.zeros((T, H, D), dtype=np.float64)
    heads = range(H) if heads is None else heads
    for i in range(len(lens)):
        a, b = int(query_start_loc[i]), int(query_start_loc[i + 1])
        S, L = b - a, int(lens[i])
        if S == 0:
            continue
        if S > L:
            raise ValueError("chunk longer than the sequence")
        K, V = gathered_kv(k_bits, v_bits, kv_dtype, tables[i], L, block_size, k_scale, v_scale)
        vis = chunk_visible(L, S)
        for h in heads:
            out[a:b, h] = attend(q[a:b, h], K[:, h, :], V[:, h, :], scale, vis)
    return out
