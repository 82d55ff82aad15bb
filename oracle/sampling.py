"""Sampled verification walks (test infrastructure only).

Two acceptance rules beyond the greedy walk of ``accept``:

1. Temperature sampling by the verifier, the tree only a hint.
   DDTree notes, section 7.2: from the root, each step picks a token with the
   target's own decoding rule (greedy or temperature sampling) and follows
   the drafted child carrying it, else stops with that token as the next
   bonus; section 7.3: since the verifier samples from its own distribution
   at every visited node, the emitted tokens are distributed exactly as
   plain autoregressive sampling from the target (lossless), whatever the
   draft proposed.
   Decoding page ("解码：采样、束搜索和推测性解码"), section "Gumbel Max技巧":
   sampling from Categorical(Softmax(h)) equals taking argmax_i (h_i + g_i)
   with g_i = -log(-log(z_i)), z_i ~ U(0, 1) drawn independently, and that
   noise can be prepared ahead of time.
   So each row's choice is argmax_v (logit_v / T + g_v); with all g = 0 it is
   the greedy argmax.

2. Stochastic per-edge acceptance ("02 · Token Tree 与 Tree Attention" §4):
   one target pass gives every node its distribution p; from the root, each
   child of the current node is accepted or rejected by the min(1, p / q)
   rule; an accepted child becomes the current node; when every child is
   rejected a correction token is sampled at the current node and the walk
   ends; at a leaf the bonus token is sampled from the leaf's p.  The
   min(1, p / q) rule is speculative sampling's: draft token x proposed from
   q is kept with probability min(1, p(x) / q(x)); after a rejection the
   target side continues from the residual norm(max(0, p - q)).  See
   ``stochastic_walk``.

Readings where the pages leave a step open (each is stated once more where
it is used):

* h = logits / T is formed in float32 as fl(x * fl(1 / T)) and the noise is
  added in float32, fl(h + g): one rounding per operation, no fused
  multiply-add, so a decision between two values is taken in the precision
  the kernel computes in.  The argmax takes the lowest index on ties and
  treats -0.0 like +0.0.
* The noise is an input, float32 [rows, vocab]; drawing it is the caller's
  business (``synth.gumbel_noise`` for the tests).
* Stochastic walk: p_r = softmax(x_r / T) over the row r's logits in float64
  (e_v = exp((x_v - max) / T), p = e / sum e); the draft's distribution
  q_r (float32 [rows, vocab]) is the one the children of row r's node were
  proposed from (one per parent, the same for all its children); u_j
  (float32, one per node) is node j's uniform draw for its accept test,
  accepted iff u_j * q(x_j) < r(x_j) in float64 with r the current target
  side distribution; siblings are tried in increasing index order, each
  rejection replacing r by norm(max(0, r - q)) (SpecInfer's sequential
  multi-candidate form of the rule; the page leaves the sibling order open);
  the correction or bonus token is a Gumbel-max sample of the current r:
  argmax_v (log r_v + g_v) over r_v > 0, in float64.
"""

from typing import Dict, List

import numpy as np

from .accept import greedy_walk


def inv_temperature(T: float) -> np.float32:
    """fl32(1 / T) for a temperature T > 0 (T itself taken as float32)."""
    return np.float32(1.0) / np.float32(T)


def perturbed_rows(rows_f32: np.ndarray, T: float, noise: np.ndarray) -> np.ndarray:
    """fl32(fl32(x * fl32(1/T)) + g), elementwise (x the logits widened to float32)."""
    x = np.asarray(rows_f32, dtype=np.float32)
    h = (x * inv_temperature(T)).astype(np.float32)
    return (h + np.asarray(noise, dtype=np.float32)).astype(np.float32)


def sampled_choice(rows_f32: np.ndarray, T: float, noise: np.ndarray) -> List[int]:
    """Gumbel-max choice of every row: lowest index of the maximum of x / T + g."""
    v = perturbed_rows(rows_f32, T, noise).astype(np.float64)  # exact widening; -0.0 == +0.0
    return [int(np.argmax(r)) for r in v]


def sample_accept(logits_rows_f32_of, noise_rows_of, T: float, node_offsets, tokens_all, parents_all,
                  max_accept: int) -> Dict[str, np.ndarray]:
    """Batched temperature-sampling walk.

    ``logits_rows_f32_of(b)`` / ``noise_rows_of(b)`` give request b's N_b + 1
    rows (row 0 the root, row 1 + i node i) as float32.  Same outputs as
    ``accept.accept``: accept_len, accepted_nodes, out_tokens (accepted tokens
    then the bonus / correction token, -1 after), row_choice [T + B], err.
    """
    node_offsets = np.asarray(node_offsets)
    B = len(node_offsets) - 1
    T_all = int(node_offsets[-1])
    accept_len = np.zeros(B, dtype=np.int32)
    accepted_nodes = np.full((B, max_accept), -1, dtype=np.int32)
    out_tokens = np.full((B, max_accept + 1), -1, dtype=np.int32)
    choice_all = np.zeros(T_all + B, dtype=np.int32)
    err = np.zeros(B, dtype=np.int32)
    for b in range(B):
        s, e = int(node_offsets[b]), int(node_offsets[b + 1])
        choice = sampled_choice(logits_rows_f32_of(b), T, noise_rows_of(b))
        choice_all[s + b: e + b + 1] = choice
        w = greedy_walk(choice, tokens_all[s:e], parents_all[s:e], max_accept)
        a = len(w["accepted"])
        accept_len[b] = a
        accepted_nodes[b, :a] = w["accepted"]
        out_tokens[b, :a] = w["accepted_tokens"]
        out_tokens[b, a] = w["bonus"]
        err[b] = w["err"]
    return dict(accept_len=accept_len, accepted_nodes=accepted_nodes, out_tokens=out_tokens,
                row_argmax=choice_all, err=err)


def softmax_f64(row_f32: np.ndarray, T: float) -> np.ndarray:
    """p = softmax(x / T) in float64 for one row (x widened exactly)."""
    x = np.asarray(row_f32, dtype=np.float64)
    e = np.exp((x - x.max()) / float(T))
    return e / e.sum()


def gumbel_sample(r: np.ndarray, g_row) -> int:
    """argmax_v (log r_v + g_v) over the support of r (lowest index on ties)."""
    score = np.full(r.shape, -np.inf)
    pos = r > 0
    score[pos] = np.log(r[pos]) + np.asarray(g_row, dtype=np.float64)[pos]
    return int(np.argmax(score))


def stochastic_walk(rows_f32: np.ndarray, T: float, q_rows: np.ndarray, u: np.ndarray, g_rows: np.ndarray,
                    tokens, parents, max_accept: int) -> Dict[str, object]:
    """Stochastic min(1, p/q) walk of one request.

    rows_f32 [N + 1, V]: target logits (row 0 the root, row 1 + i node i);
    q_rows [N + 1, V]: draft distribution for the children of each row's node;
    u [N]: uniform per node; g_rows [N + 1, V]: Gumbel noise per row.
    Returns accepted nodes, their tokens, the final (correction / bonus)
    token and err bits (16 when an acceptance would exceed max_accept).
    """
    tokens = [int(t) for t in tokens]
    parents = [int(p) for p in parents]
    n = len(parents)
    accepted: List[int] = []
    err = 0
    cur, row = -1, 0
    r = softmax_f64(rows_f32[0], T)
    while True:
        children = [j for j in range(n) if parents[j] == cur]
        q = np.asarray(q_rows[row], dtype=np.float64)
        nxt = None
        for j in children:
            x = tokens[j]
            if float(np.float64(u[j]) * q[x]) < r[x]:
                nxt = j
                break
            res = np.maximum(r - q, 0.0)
            z = res.sum()
            if z > 0:
                r = res / z
        if nxt is None:
            return dict(accepted=accepted, accepted_tokens=[tokens[j] for j in accepted],
                        bonus=gumbel_sample(r, g_rows[row]), err=err)
        if len(accepted) == max_accept:
            err |= 16
            return dict(accepted=accepted, accepted_tokens=[tokens[j] for j in accepted], bonus=-1, err=err)
        accepted.append(nxt)
        cur, row = nxt, 1 + nxt
        r = softmax_f64(rows_f32[row], T)


def stochastic_accept(logits_rows_f32_of, q_rows_of, u_all, g_rows_of, T: float, node_offsets, tokens_all,
                      parents_all, max_accept: int) -> Dict[str, np.ndarray]:
    """Batched stochastic walk, outputs shaped like ``accept.accept`` (no row choices)."""
    node_offsets = np.asarray(node_offsets)
    B = len(node_offsets) - 1
    accept_len = np.zeros(B, dtype=np.int32)
    accepted_nodes = np.full((B, max_accept), -1, dtype=np.int32)
    out_tokens = np.full((B, max_accept + 1), -1, dtype=np.int32)
    err = np.zeros(B, dtype=np.int32)
    for b in range(B):
        s, e = int(node_offsets[b]), int(node_offsets[b + 1])
        w = stochastic_walk(logits_rows_f32_of(b), T, q_rows_of(b), u_all[s:e], g_rows_of(b),
                            tokens_all[s:e], parents_all[s:e], max_accept)
        a = len(w["accepted"])
        accept_len[b] = a
        accepted_nodes[b, :a] = w["accepted"]
        out_tokens[b, :a] = w["accepted_tokens"]
        out_tokens[b, a] = w["bonus"] if a < max_accept + 1 else -1
        err[b] = w["err"]
    return dict(accept_len=accept_len, accepted_nodes=accepted_nodes, out_tokens=out_tokens, err=err)
