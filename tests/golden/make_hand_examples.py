"""Writes hand_examples.json: three tiny NHA cases worked out by hand.

Each value below is the closed form derived step by step in the 'derivation'
strings (the K^long_t recurrence with the token shift, and one softmax over
slots + window, as defined on the Paper-Notes page 'Native Hybrid Attention for
Efficient Sequence Modeling', section 关键设计 > 层内混合).  Only math.exp /
log / sin / cos of small literals are evaluated; no oracle or kernel is called.
Run from the repository root:  python tests/golden/make_hand_examples.py
"""
import json
import math
import os

e = math.e
k = [[1, 0], [0, 1], [1, 1]]
v = [[1, 0], [0, 2], [3, 0]]
q = [[1, 0], [0, 1], [1, 1]]


def sm(ls):
    M = max(ls)
    es = [math.exp(x - M) for x in ls]
    Z = sum(es)
    return [x / Z for x in es], M + math.log(Z)


cases = []
# case A: d=2, m=1, w=1, alpha=0.5, scale=1, no RoPE
a, b = math.exp(0.75), math.exp(2.0)
cases.append({
    "name": "w1_norope", "B": 1, "T": 3, "H": 1, "Hkv": 1, "d": 2, "m": 1, "w": 1,
    "rope_base": 0.0, "scale": 1.0, "q": q, "k": k, "v": v, "alpha": [[0.5]] * 3,
    "derivation": [
        "t=0: slots zero; logits [0, q0.k0=1] -> o0=e/(1+e) v0, lse=ln(1+e)",
        "t=1: absorb k0,v0 with alpha_1: SK=(0.5,0), SV=(0.5,0); logits [q1.SK=0, q1.k1=1] -> o1=(0.5/(1+e), 2e/(1+e)), lse=ln(1+e)",
        "t=2: absorb k1,v1 with alpha_2: SK=(0.25,0.5), SV=(0.25,1); logits [0.75, 2] -> o2=(e^0.75 (0.25,1) + e^2 (3,0))/(e^0.75+e^2)"],
    "o": [[e / (1 + e), 0.0], [0.5 / (1 + e), 2 * e / (1 + e)],
          [(a * 0.25 + b * 3) / (a + b), a / (a + b)]],
    "lse": [math.log(1 + e), math.log(1 + e), math.log(a + b)]})

# case B: same tokens, w=2, RoPE on; d=2 -> theta_0 = 1 rad per position for any base
s1, c1 = math.sin(1.0), math.cos(1.0)
l_a, l_b = -s1, 1.0
Z1 = 1.0 + math.exp(l_a) + math.exp(l_b)
l_s, l_1, l_2 = 0.5, s1 + c1, 2.0
Z2 = math.exp(l_s) + math.exp(l_1) + math.exp(l_2)
cases.append({
    "name": "w2_rope", "B": 1, "T": 3, "H": 1, "Hkv": 1, "d": 2, "m": 1, "w": 2,
    "rope_base": 10000.0, "scale": 1.0, "q": q, "k": k, "v": v, "alpha": [[0.5]] * 3,
    "derivation": [
        "d=2 so theta_0 = base^0 = 1: R_t rotates by t radians; <R_t q, R_j k> = <q, R_{j-t} k>",
        "t=0: window {0}: logit 1, slots zero -> o0=e/(1+e) v0",
        "t=1: window {0,1}: <q1, R_{-1} k0> = -sin 1, <q1,k1> = 1; slots still zero (t<w)",
        "t=2: absorb k0,v0 with alpha_2 -> SK=SV=(0.5,0); slot logit 0.5; window {1,2}: <q2, R_{-1} k1> = sin1+cos1, <q2,k2> = 2"],
    "o": [[e / (1 + e), 0.0],
          [math.exp(l_a) / Z1, 2.0 * math.exp(l_b) / Z1],
          [(0.5 * math.exp(l_s) + 3.0 * math.exp(l_2)) / Z2, 2.0 * math.exp(l_1) / Z2]],
    "lse": [math.log(1 + e), math.log(Z1), math.log(Z2)]})

# case C: w=0 (pure linear RNN read by a softmax over the slots), m=2, gates 0.5 and 0
rows = [([0.5, 0.0], [1.0, 0.0], [0.5, 0.0], [1.0, 0.0], [0.5, 1.0]),
        ([0.25, 0.5], [0.0, 1.0], [0.25, 1.0], [0.0, 2.0], [0.5, 1.0]),
        ([0.625, 0.75], [1.0, 1.0], [1.625, 0.5], [3.0, 0.0], [1.375, 2.0])]
oC, lC = [], []
for SK0, SK1, SV0, SV1, logits in rows:
    p, l = sm(logits)
    oC.append([p[0] * SV0[0] + p[1] * SV1[0], p[0] * SV0[1] + p[1] * SV1[1]])
    lC.append(l)
cases.append({
    "name": "w0_two_slots", "B": 1, "T": 3, "H": 1, "Hkv": 1, "d": 2, "m": 2, "w": 0,
    "rope_base": 0.0, "scale": 1.0, "q": q, "k": k, "v": v, "alpha": [[0.5, 0.0]] * 3,
    "derivation": [
        "w=0: empty window; token t is absorbed at step t before the read",
        "slot 0 has gate 0.5, slot 1 gate 0 (it always equals the current token)",
        "t=0: SK=[(0.5,0),(1,0)], SV=[(0.5,0),(1,0)], logits [0.5,1]",
        "t=1: SK=[(0.25,0.5),(0,1)], SV=[(0.25,1),(0,2)], logits [0.5,1]",
        "t=2: SK=[(0.625,0.75),(1,1)], SV=[(1.625,0.5),(3,0)], logits [1.375,2]"],
    "o": oC, "lse": lC})

out = {"citation": ("Hand-derived from the K^long_t recurrence and the o_t formula of the "
                    "Paper-Notes page 'Native Hybrid Attention for Efficient Sequence Modeling', "
                    "section 关键设计 > 层内混合, with its token shift (token t-w enters the slots "
                    "at step t with gate alpha_t). The pages print no worked example."),
       "cases": cases}
with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "hand_examples.json"), "w") as f:
    json.dump(out, f, indent=1, ensure_ascii=False)
