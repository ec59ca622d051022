"""Writes the hand-derived oracle pins in this folder (run: python write_hand_cases.py).

Every expected value here is worked out by hand from the definition (see each
case's ``derivation``); the script calls no implementation, it only evaluates the
log() constants used as table entries and writes JSON.

Definition followed (prhub page for vllm-project/vllm PR #55629, section
关键源码片段): row-major tokens ``i = qh*W + qw``; ``rel_h[i,kh] = q_i . T_h[qh-kh+H-1]``
and ``rel_w[i,kw] = q_i . T_w[qw-kw+W-1]`` on the unscaled q; dense bias
``rel_h[i, j//W] + rel_w[i, j%W]``; ``out = softmax(scale*q.k + bias) @ v``.
"""

import json
import math
import os

LN2, LN3 = math.log(2.0), math.log(3.0)
CITE = ("prhub page for vllm-project/vllm PR #55629 (DeepEncoder relative-position "
        "attention fused into a Triton kernel), section 关键源码片段: tokens are the "
        "row-major H*W grid, add_decomposed_rel_pos(q, rel_pos_h, rel_pos_w, (H,W), (H,W)) "
        "on the unscaled q, SDPA with the dense (rel_h + rel_w) bias; table index qh-kh+H-1 "
        "and qw-kw+W-1 is the reading taken of the helper the page does not print.")

CASES = [
    dict(name="index_sign_2x2", H=2, W=2, scale=0.125,
         q=[[1.0]] * 4, k=[[0.0]] * 4, v=[[1.0], [2.0], [3.0], [4.0]],
         rel_pos_h=[[0.0], [0.0], [LN3]], rel_pos_w=[[0.0], [0.0], [0.0]],
         expected_rel_h=[[0.0, 0.0], [0.0, 0.0], [LN3, 0.0], [LN3, 0.0]],
         expected_rel_w=[[0.0, 0.0]] * 4,
         expected_out=[[2.5], [2.5], [2.0], [2.0]],
         derivation=("k=0 so scores are the bias alone. rel_h[i,kh]=T_h[qh-kh+1]: qh=0 -> [T1,T0]=[0,0], "
                     "so rows 0,1 are uniform: mean(1,2,3,4)=2.5. qh=1 -> [T2,T1]=[ln3,0]: keys 0,1 (kh=0) "
                     "weigh 3, keys 2,3 weigh 1: (3*1+3*2+3+4)/8=2. The flipped index kh-qh+1 would give "
                     "[3,3,2.5,2.5]; scaling q by 1/8 before the bias gives about 2.43 on rows 2,3.")),
    dict(name="flatten_axes_2x3", H=2, W=3, scale=0.125,
         q=[[1.0]] * 6, k=[[0.0]] * 6, v=[[0.0], [1.0], [2.0], [3.0], [4.0], [5.0]],
         rel_pos_h=[[0.0]] * 3, rel_pos_w=[[LN2], [0.0], [0.0], [0.0], [0.0]],
         expected_rel_h=[[0.0, 0.0]] * 6,
         expected_rel_w=[[0.0, 0.0, LN2], [0.0, 0.0, 0.0], [0.0, 0.0, 0.0],
                         [0.0, 0.0, LN2], [0.0, 0.0, 0.0], [0.0, 0.0, 0.0]],
         expected_out=[[2.75], [2.5], [2.5], [2.75], [2.5], [2.5]],
         derivation=("rel_w[i,kw]=T_w[qw-kw+2] is ln2 only for qw=0,kw=2. Queries 0 and 3 (qw=0) weigh "
                     "keys 2 and 5 (kw=2) by 2: (0+1+2*2+3+4+2*5)/8=22/8=2.75; the rest are uniform: 15/6=2.5. "
                     "Column-major flattening would move the weighted keys and give 3 on row 0.")),
    dict(name="scale_on_qk_1x2", H=1, W=2, scale=0.125,
         q=[[1.0], [1.0]], k=[[0.0], [8.0 * LN3]], v=[[0.0], [4.0]],
         rel_pos_h=[[0.0]], rel_pos_w=[[0.0], [0.0], [0.0]],
         expected_rel_h=[[0.0], [0.0]], expected_rel_w=[[0.0, 0.0], [0.0, 0.0]],
         expected_out=[[3.0], [3.0]],
         derivation=("Tables are zero. scale*q.k = [0, ln3], weights 1:3, out=(0+3*4)/4=3 for both queries. "
                     "Dropping the scale gives weights 1:3^8.")),
    dict(name="unscaled_q_in_bias_1x2", H=1, W=2, scale=0.125,
         q=[[2.0], [2.0]], k=[[0.0], [0.0]], v=[[0.0], [4.0]],
         rel_pos_h=[[0.0]], rel_pos_w=[[LN3 / 2.0], [0.0], [0.0]],
         expected_rel_h=[[0.0], [0.0]], expected_rel_w=[[0.0, LN3], [0.0, 0.0]],
         expected_out=[[3.0], [2.0]],
         derivation=("rel_w[0,1]=q*T_w[0-1+1]=2*(ln3/2)=ln3, all else 0. Query 0 weighs key 1 by 3: "
                     "(0+3*4)/4=3; query 1 is uniform: 2. With q scaled by 1/8 in the bias, query 0 "
                     "would give 4*3^(1/8)/(1+3^(1/8)) ~= 2.137.")),
    dict(name="both_axes_2x2_d2", H=2, W=2, scale=0.125,
         q=[[1.0, 1.0]] * 4, k=[[0.0, 0.0]] * 4, v=[[1.0, 0.0], [2.0, 0.0], [3.0, 0.0], [4.0, 8.0]],
         rel_pos_h=[[0.0, 0.0], [0.0, 0.0], [LN2, 0.0]], rel_pos_w=[[0.0, LN3], [0.0, 0.0], [0.0, 0.0]],
         expected_rel_h=[[0.0, 0.0], [0.0, 0.0], [LN2, 0.0], [LN2, 0.0]],
         expected_rel_w=[[0.0, LN3], [0.0, 0.0], [0.0, LN3], [0.0, 0.0]],
         expected_out=[[2.75, 3.0], [2.5, 2.0], [29.0 / 12.0, 2.0], [13.0 / 6.0, 4.0 / 3.0]],
         derivation=("rel_h: qh=1,kh=0 -> ln2; rel_w: qw=0,kw=1 -> ln3 (dot with q=(1,1) sums the row). "
                     "Key weights (keys (0,0),(0,1),(1,0),(1,1)): q0 [1,3,1,3]/8 -> (22/8, 24/8); "
                     "q1 uniform -> (10/4, 8/4); q2 [2,6,1,3]/12 -> (29/12, 24/12); q3 [2,2,1,1]/6 -> (13/6, 8/6).")),
]


def main():
    here = os.path.dirname(os.path.abspath(__file__))
    for c in CASES:
        c = dict(c, citation=CITE)
        with open(os.path.join(here, c["name"] + ".json"), "w") as f:
            json.dump(c, f, indent=1)


if __name__ == "__main__":
    main()
