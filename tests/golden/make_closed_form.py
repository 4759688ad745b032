"""Writes attention_closed_form.json: hand-derived attention cases.

Every expected value in the fixture is an exact fraction derived by hand (the
derivation travels with each fixture); this script calls nothing from the
oracle or the HIP library.  Inputs use logs of small integers so that the
softmax weights are exact rationals.  Definition followed: bidirectional
attention softmax(Q K^T * scale) V per image and head over the kept tokens
("Dispatch-Aware Ragged Attention for Pruned Vision Transformers", sota2.com
page, Abstract; aissential.tech summary, Method).
"""
import json
import math
import os

ln2, ln3, ln4 = math.log(2), math.log(3), math.log(4)
BIG = 1000.0
CITATION = ("Dispatch-Aware Ragged Attention for Pruned Vision Transformers (arXiv 2604.15408): "
            "sota2.com page, Abstract (pack-attend-unpack pipeline around bidirectional attention "
            "over variable-length sequences); aissential.tech summary, Method. The formula "
            "softmax(Q K^T * scale) V per image and head is the plain reading of 'bidirectional "
            "attention'.")


def F(a, b=1):
    return [a, b]


def fixture_scale_one():
    mask = [[1, 0, 1, 1], [1, 1, 0, 0], [0, 0, 0, 0]]
    r = lambda x: [x]  # one head
    q = [[r([1, 0]), r([BIG, -BIG]), r([0, 0]), r([2, 0])],
         [r([0, 1]), r([0, -1]), r([BIG, BIG]), r([-BIG, 3])],
         [r([BIG, 0]), r([0, BIG]), r([1, 1]), r([-1, -1])]]
    k = [[r([0, 0]), r([BIG, BIG]), r([ln2, 0]), r([ln3, 0])],
         [r([0, ln4]), r([0, 0]), r([-BIG, 0]), r([BIG, 1])],
         [r([1, 2]), r([3, 4]), r([5, 6]), r([7, 8])]]
    v = [[r([1, 0]), r([BIG, BIG]), r([0, 1]), r([1, 1])],
         [r([10, -5]), r([0, 5]), r([BIG, -BIG]), r([7, 7])],
         [r([1, 1]), r([1, 1]), r([1, 1]), r([1, 1])]]
    Z = [F(0), F(0)]
    expected = [[[[F(2, 3), F(5, 6)]], [Z], [[F(2, 3), F(2, 3)]], [[F(5, 7), F(13, 14)]]],
                [[[F(8), F(-3)]], [[F(2), F(3)]], [Z], [Z]],
                [[Z], [Z], [Z], [Z]]]
    return {
        "citation": CITATION,
        "derivation": [
            "Image 0 keeps tokens 0,2,3. Keys (ln1,0),(ln2,0),(ln3,0), scale 1.",
            "Query (1,0): logits 0, ln2, ln3 -> weights 1/6, 2/6, 3/6; V rows (1,0),(0,1),(1,1) -> O = (2/3, 5/6).",
            "Query (0,0): uniform 1/3 -> O = (2/3, 2/3).",
            "Query (2,0): logits 0, 2ln2, 2ln3 -> weights 1/14, 4/14, 9/14 -> O = (5/7, 13/14).",
            "Image 1 keeps tokens 0,1. Keys (0,ln4),(0,0). Query (0,1): logits ln4, 0 -> 4/5, 1/5; V (10,-5),(0,5) -> (8,-3).",
            "Query (0,-1): logits -ln4, 0 -> 1/5, 4/5 -> (2, 3).",
            "Image 2 keeps nothing: all its output rows are +0. Pruned rows everywhere are +0.",
            "Pruned positions hold +-1000 so a leak across the mask or across images changes the result.",
            "K Q^T in place of Q K^T gives different weights for image 0 (its keys and queries differ).",
        ],
        "B": 3, "N": 4, "H": 1, "d": 2, "scale": 1.0,
        "mask": mask, "q": q, "k": k, "v": v,
        "expected_cu_seqlens": [0, 3, 5, 5], "expected_max_seqlen": 3,
        "expected_kept_index": [0, 2, 3, 4, 5],
        "expected_o_fraction": expected,
    }


def fixture_default_scale():
    q = [[[[1, 0, 0, 0], [1, 0, 0, 0]], [[0, 0, 0, 0], [0, 0, 0, 0]], [[2, 0, 0, 0], [0, 0, 0, 0]]]]
    k = [[[[0, 0, 0, 0], [2 * ln3, 0, 0, 0]], [[2 * ln2, 0, 0, 0], [2 * ln2, 0, 0, 0]],
          [[2 * ln3, 0, 0, 0], [0, 0, 0, 0]]]]
    v = [[[[6, 0, 0, 0], [6, 0, 0, -6]], [[0, 6, 0, 0], [0, 6, 0, 6]], [[0, 0, 6, 0], [0, 0, 6, 0]]]]
    expected = [[[[F(1), F(2), F(3), F(0)], [F(3), F(2), F(1), F(-1)]],
                 [[F(2), F(2), F(2), F(0)], [F(2), F(2), F(2), F(0)]],
                 [[F(3, 7), F(12, 7), F(27, 7), F(0)], [F(2), F(2), F(2), F(0)]]]]
    return {
        "citation": CITATION + " Scale 1/sqrt(d) is the standard scaled dot-product reading.",
        "derivation": [
            "d = 4, default scale 1/2. Head 0 keys (2 ln(j+1),0,0,0): query (1,0,0,0) has scaled logits 0, ln2, ln3 -> weights 1/6,1/3,1/2 -> O = (1,2,3,0).",
            "Head 0 query 0 -> uniform -> (2,2,2,0); query (2,0,0,0) -> weights 1/14,4/14,9/14 -> (3/7,12/7,27/7,0).",
            "Head 1 keys reversed: query (1,0,0,0) -> weights 1/2,1/3,1/6 over V rows (6,0,0,-6),(0,6,0,6),(0,0,6,0) -> (3,2,1,-1).",
            "Head 1 queries 0 -> uniform -> (2,2,2,0).",
            "A missing scale or a 1/d scale changes head 0 query (1,0,0,0).",
        ],
        "B": 1, "N": 3, "H": 2, "d": 4, "scale": None,
        "mask": [[1, 1, 1]], "q": q, "k": k, "v": v,
        "expected_cu_seqlens": [0, 3], "expected_max_seqlen": 3, "expected_kept_index": [0, 1, 2],
        "expected_o_fraction": expected,
    }


if __name__ == "__main__":
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "attention_closed_form.json")
    with open(out, "w") as f:
        json.dump({"fixtures": [fixture_scale_one(), fixture_default_scale()]}, f, indent=1)
    print("wrote", out)
