"""Writes hand_examples.json: four tiny NHA cases worked out by hand.

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

# case D: d=8, base=16 -> theta_i = 16^(-2i/8) = 2^-i exactly (1, 1/2, 1/4, 1/8);
# rotate-half pairs (i, i+4).  w=3 >= T: every token stays in the window, the
# single slot is never written (logit 0, value 0).  The weights 1..4 on the
# four frequencies and keys with their mass in the second half fix the
# frequency of every pair, the pairing and the direction of the rotation.
e8 = lambda i, x=1.0: [x if j == i else 0.0 for j in range(8)]
qD = [e8(0), e8(4), [1.0, 2.0, 3.0, 4.0, 0.0, 0.0, 0.0, 0.0]]
kD = [[1.0, 1.0, 1.0, 1.0, 0.0, 0.0, 0.0, 0.0], [0.0, 0.0, 0.0, 0.0, 1.0, 1.0, 1.0, 1.0], e8(0)]
vD = [e8(0, 1.0), e8(1, 2.0), e8(2, 3.0)]
th = [1.0, 0.5, 0.25, 0.125]
# t=1: key 0 at relative position -1: only pair (0, 4) meets q1 = e_4
l10, l11 = -math.sin(1.0), 0.0
# t=2: key 0 at -2: sum_i (i+1) cos(2 theta_i); key 1 at -1: sum_i (i+1) sin(theta_i); key 2: q2.k2 = 1
l20 = sum((i + 1) * math.cos(2 * th[i]) for i in range(4))
l21 = sum((i + 1) * math.sin(th[i]) for i in range(4))
l22 = 1.0
Z0 = 1.0 + e
Z1 = 1.0 + math.exp(l10) + math.exp(1.0)
Z2 = 1.0 + math.exp(l20) + math.exp(l21) + math.exp(l22)
oD = [[x * e / Z0 for x in vD[0]],
      [(math.exp(l10) * a0 + math.exp(1.0) * a1) / Z1 for a0, a1 in zip(vD[0], vD[1])],
      [(math.exp(l20) * a0 + math.exp(l21) * a1 + math.exp(l22) * a2) / Z2 for a0, a1, a2 in zip(*vD)]]
cases.append({
    "name": "d8_rope_frequencies", "B": 1, "T": 3, "H": 1, "Hkv": 1, "d": 8, "m": 1, "w": 3,
    "rope_base": 16.0, "scale": 1.0, "q": qD, "k": kD, "v": vD, "alpha": [[0.5]] * 3,
    "derivation": [
        "theta_i = 16^(-2i/8) = 2^-i: 1, 1/2, 1/4, 1/8 rad per position; pairs (i, i+4)",
        "R_a^T R_b = R_(b-a), so <R_t q, R_j k> = <q, R_(j-t) k>; R_phi maps (x_i, x_(i+4)) to "
        "(x_i cos(phi theta_i) - x_(i+4) sin(phi theta_i), x_(i+4) cos(phi theta_i) + x_i sin(phi theta_i))",
        "t=0: window {0}: <e_0, k0> = 1 -> o0 = e/(1+e) v0",
        "t=1: window {0,1}: <e_4, R_-1 k0> = k0_0 sin(-1) = -sin 1 ; <e_4, k1> = 1",
        "t=2: window {0,1,2}: <q2, R_-2 k0> = sum_i (i+1) cos(2 theta_i); "
        "<q2, R_-1 k1> = sum_i (i+1) (-k1_(i+4)) sin(-theta_i) = sum_i (i+1) sin(theta_i); <q2, k2> = 1",
        "slot: never written (t < w for every t): logit 0, value 0, it only adds 1 to Z"],
    "o": oD, "lse": [math.log(Z0), math.log(Z1), math.log(Z2)]})

out = {"citation": ("Hand-derived from the K^long_t recurrence and the o_t formula of the "
                    "Paper-Notes page 'Native Hybrid Attention for Efficient Sequence Modeling', "
                    "section 关键设计 > 层内混合, with its token shift (token t-w enters the slots "
                    "at step t with gate alpha_t). The pages print no worked example."),
       "cases": cases}
with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "hand_examples.json"), "w") as f:
    json.dump(out, f, indent=1, ensure_ascii=False)
