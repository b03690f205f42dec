"""Writes hand_4x4.json: a 4x4 attention case worked out on paper.

The values are closed forms of the derivation below; this script evaluates them and
calls neither the oracle nor the HIP library. Definition used: softmax(Q K^T * scale
+ mask) V ("Flash MSA Attention Kernel Implementation: A Practical Guide for
Production AI", section "Why Standard Attention Broke"); causal masking of keys after
the query (same page, CUDA forward kernel section); the backward equations of the same
page's section "The Backward Pass: The Real Beast", with the scale from the chain rule.

Run from the repository root: python tests/golden/make_hand_4x4.py
"""
import json
import math
import os

LN3 = math.log(3.0)

DERIVATION = [
    "d=4, scale=1, Q = I, K = ln(3) I, V = 6 I, so S = ln(3) I.",
    "Non-causal: exp(S) has 3 on the diagonal and 1 elsewhere; row sum 6; P_ii = 1/2, "
    "P_ij = 1/6; O = 6 P; LSE_i = ln 6.",
    "Causal: row i sees keys 0..i with weights 1 (j<i) and 3 (j=i); row sum i+3; "
    "O_i = 6 P_i; LSE_i = ln(i+3).",
    "Backward with dO = I: dP = dO V^T = 6 I; D_i = sum_j P_ij dP_ij = 6 P_ii; "
    "dS = P o (dP - D); dQ = scale dS K = ln(3) dS; dK = scale dS^T Q = dS^T; dV = P^T dO = P^T.",
    "Non-causal: D_i = 3, dS_ii = 1.5, dS_ij = -0.5.",
    "Causal: P_ii = 3/(i+3), P_ij = 1/(i+3) for j<i; D_i = 18/(i+3); dS_ii = P_ii (6 - D_i); "
    "dS_ij = -P_ij D_i for j<i; dS_ij = 0 for j>i.",
]


def probs(causal):
    P = [[0.0] * 4 for _ in range(4)]
    for i in range(4):
        den = (i + 3) if causal else 6
        for j in range(4):
            if causal and j > i:
                continue
            P[i][j] = (3.0 if i == j else 1.0) / den
    return P


def backward(causal):
    P = probs(causal)
    dS = [[P[i][j] * ((6.0 if i == j else 0.0) - 6.0 * P[i][i]) for j in range(4)] for i in range(4)]
    dQ = [[LN3 * dS[i][j] for j in range(4)] for i in range(4)]
    dK = [[dS[j][i] for j in range(4)] for i in range(4)]
    dV = [[P[j][i] for j in range(4)] for i in range(4)]
    return {"dQ": dQ, "dK": dK, "dV": dV}


def main():
    out = {
        "source": "hand derivation (closed forms); see make_hand_4x4.py",
        "derivation": DERIVATION,
        "inputs": {"scale": 1.0, "Q": "identity(4)", "K": "ln(3) * identity(4)",
                   "V": "6 * identity(4)", "dO": "identity(4)"},
        "noncausal": {"O": [[6.0 * p for p in row] for row in probs(False)],
                      "LSE": [math.log(6.0)] * 4},
        "causal": {"O": [[6.0 * p for p in row] for row in probs(True)],
                   "LSE": [math.log(i + 3.0) for i in range(4)]},
        "noncausal_bwd": backward(False),
        "causal_bwd": backward(True),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hand_4x4.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
