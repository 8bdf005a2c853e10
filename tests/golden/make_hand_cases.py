"""Writes hand_cases.json: hand-derived worked examples of attention.

The source pages print no numeric worked example, so these cases are built by
hand: every score is the logarithm of a small integer, which makes each
softmax weight an exact rational and each output a short sum that the
'derivation' field spells out.  This script calls nothing: it only writes the
hand-derived numbers (ln 2 and ln 3 to full double precision).

Definitions followed: "Triton Ascend Attention", section "standard attention
computation flow" (scaled scores, row softmax summing to one, weighted sum
with V); the FlashAttention-2 forward article's kernel epilogue (the stored
row statistic is m + log(l), natural log); causal masking keeps the diagonal
("flash-attention-kernel" skill page, pitfalls; the article's _attn_fwd_inner
mask), counted from the top-left corner.

Run: python tests/golden/make_hand_cases.py
"""
import json
import math
import os

L2, L3 = math.log(2.0), math.log(3.0)
CITE_DEF = ("Triton Ascend Attention, 'standard attention computation flow' "
            "(three phases: scaled scores, row softmax summing to one, "
            "weighted sum with V); FlashAttention-2 forward article "
            "(wsisp.com), kernel epilogue storing m + log(l) per row")
CITE_CAUSAL = ("flash-attention-kernel skill page, pitfalls (offs_m >= offs_n "
               "keeps the diagonal); FlashAttention-2 forward article, "
               "_attn_fwd_inner causal mask")

K3 = [[[[0.0], [L2], [L3]]]]
V3 = [[[[6.0], [12.0], [18.0]]]]

CASES = [
    dict(name="three_keys_one_query", cite=CITE_DEF,
         derivation="scores = q*k = [0, ln2, ln3]; exp = [1,2,3], sum 6; "
                    "P = [1/6,1/3,1/2]; O = 6/6 + 12/3 + 18/2 = 14; LSE = ln 6",
         B=1, H=1, Lq=1, Lk=3, D=1, causal=False, scale=1.0,
         q=[[[[1.0]]]], k=K3, v=V3, o=[[[[14.0]]]], lse=[[[math.log(6.0)]]]),
    dict(name="causal_three_queries", cite=CITE_DEF + "; " + CITE_CAUSAL,
         derivation="row 0 sees key 0: O = 6, LSE = 0; row 1 sees keys 0,1: "
                    "exp = [1,2], P = [1/3,2/3], O = 2 + 8 = 10, LSE = ln 3; "
                    "row 2 sees all: O = 14, LSE = ln 6",
         B=1, H=1, Lq=3, Lk=3, D=1, causal=True, scale=1.0,
         q=[[[[1.0], [1.0], [1.0]]]], k=K3, v=V3,
         o=[[[[6.0], [10.0], [14.0]]]],
         lse=[[[0.0, math.log(3.0), math.log(6.0)]]]),
    dict(name="noncausal_three_queries", cite=CITE_DEF,
         derivation="every row sees all three keys: O = 14, LSE = ln 6",
         B=1, H=1, Lq=3, Lk=3, D=1, causal=False, scale=1.0,
         q=[[[[1.0], [1.0], [1.0]]]], k=K3, v=V3,
         o=[[[[14.0], [14.0], [14.0]]]], lse=[[[math.log(6.0)] * 3]]),
    dict(name="two_dim_dot_half_scale", cite=CITE_DEF,
         derivation="scale*q = [1,2]; scores = k_x + 2 k_y = [0, ln2, ln3, "
                    "2 ln2]; exp = [1,2,3,4], sum 10; P = [.1,.2,.3,.4]; "
                    "O = [1 + 0 + 3 - 4, 0 + 2 + 3 + 2] = [0, 7]; LSE = ln 10",
         B=1, H=1, Lq=1, Lk=4, D=2, causal=False, scale=0.5,
         q=[[[[2.0, 4.0]]]],
         k=[[[[0.0, 0.0], [L2, 0.0], [L3, 0.0], [0.0, L2]]]],
         v=[[[[10.0, 0.0], [0.0, 10.0], [10.0, 10.0], [-10.0, 5.0]]]],
         o=[[[[0.0, 7.0]]]], lse=[[[math.log(10.0)]]]),
    dict(name="two_heads", cite=CITE_DEF,
         derivation="head 0: scores [0, ln3], exp [1,3], P [1/4,3/4], "
                    "O = 1 + 6 = 7, LSE = ln 4; head 1: scores 2*[ln2, 0] = "
                    "[ln4, 0], exp [4,1], P [.8,.2], O = 4 + 2 = 6, LSE = ln 5",
         B=1, H=2, Lq=1, Lk=2, D=1, causal=False, scale=1.0,
         q=[[[[1.0]], [[2.0]]]], k=[[[[0.0], [L3]], [[L2], [0.0]]]],
         v=[[[[4.0], [8.0]], [[5.0], [10.0]]]],
         o=[[[[7.0]], [[6.0]]]], lse=[[[math.log(4.0)], [math.log(5.0)]]]),
    dict(name="causal_fewer_queries_than_keys",
         cite=CITE_DEF + "; " + CITE_CAUSAL,
         derivation="top-left alignment: row 0 sees key 0 (O = 6, LSE = 0); "
                    "row 1 sees keys 0,1 (O = 10, LSE = ln 3); key 2 is never "
                    "visible",
         B=1, H=1, Lq=2, Lk=3, D=1, causal=True, scale=1.0,
         q=[[[[1.0], [1.0]]]], k=K3, v=V3, o=[[[[6.0], [10.0]]]],
         lse=[[[0.0, math.log(3.0)]]]),
    dict(name="causal_more_queries_than_keys",
         cite=CITE_DEF + "; " + CITE_CAUSAL,
         derivation="top-left alignment: rows 0,1 as before; rows 2 and 3 see "
                    "all three keys (O = 14, LSE = ln 6)",
         B=1, H=1, Lq=4, Lk=3, D=1, causal=True, scale=1.0,
         q=[[[[1.0], [1.0], [1.0], [1.0]]]], k=K3, v=V3,
         o=[[[[6.0], [10.0], [14.0], [14.0]]]],
         lse=[[[0.0, math.log(3.0), math.log(6.0), math.log(6.0)]]]),
]

if __name__ == "__main__":
    doc = {"about": "Hand-derived worked examples (see make_hand_cases.py).",
           "cases": CASES}
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                       "hand_cases.json")
    with open(out, "w") as f:
        json.dump(doc, f, indent=1)
    print(out)
