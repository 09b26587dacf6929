"""Dense fp64 tree-WY solve with numpy -- an independent route to the same numbers.

Unrolling the gated delta rule along a root-to-node path (page "Trees from
Marginals: Autoregressive drafting with factorized priors", section 3: the
state-update equation, the interaction matrices X and Y over ancestor
relations and the linear system (I + X) U = beta V) gives, with
Gamma_i = sum of ln g over node i's path (inclusive) and u_i the rank-one
write of node i:

    S_i = e^{Gamma_i} S0 + sum_{j in anc*(i)} e^{Gamma_i - Gamma_j} u_j k_j^T
    (I + X) U = R,   X_ij = beta_i e^{Gamma_i-Gamma_j} k_i.k_j  (j strict ancestor)
                     R    = diag(beta) (V - diag(e^Gamma) K S0^T)
    O = diag(e^Gamma) Q S0^T + Y U,  Y_ij = e^{Gamma_i-Gamma_j} q_i.k_j (j in anc*(i))

The page prints only the S0 = 0, undecayed right-hand side beta V.  This file
solves the full system with numpy.linalg.solve; tests compare it with the
path-walking oracle.  It shares no code with the oracle or the HIP library.
"""
import numpy as np


def ancestors(parent, i):
    out = []
    j = parent[i]
    while j >= 0:
        out.append(j)
        j = parent[j]
    return out


def solve_unit(S0, K, Q, V, beta, g, parent, accepted):
    """One (sequence, value head) unit.  S0 [dv][dk], K/Q [N][dk], V [N][dv],
    beta/g [N], parent [N].  Returns o [N][dv], u [N][dv], Gamma [N], S_acc."""
    N = len(parent)
    anc = [ancestors(parent, i) for i in range(N)]
    lg = np.log(g)
    Gam = np.array([lg[i] + sum(lg[j] for j in anc[i]) for i in range(N)])
    X = np.zeros((N, N))
    Y = np.zeros((N, N))
    for i in range(N):
        Y[i, i] = Q[i] @ K[i]
        for j in anc[i]:
            X[i, j] = beta[i] * np.exp(Gam[i] - Gam[j]) * (K[i] @ K[j])
            Y[i, j] = np.exp(Gam[i] - Gam[j]) * (Q[i] @ K[j])
    eG = np.exp(Gam)[:, None]
    R = beta[:, None] * (V - eG * (K @ S0.T))
    U = np.linalg.solve(np.eye(N) + X, R)
    O = eG * (Q @ S0.T) + Y @ U
    if accepted < 0:
        S_acc = S0.copy()
    else:
        a = accepted
        S_acc = np.exp(Gam[a]) * S0
        for j in [a] + anc[a]:
            S_acc = S_acc + np.exp(Gam[a] - Gam[j]) * np.outer(U[j], K[j])
    return O, U, Gam, S_acc
