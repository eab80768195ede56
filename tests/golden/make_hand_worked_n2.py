"""Writes hand_worked_n2.json: two tiny cases whose every output is derived by hand.

The MegaFold pages print no numeric worked example for the attention operator,
so these fixtures are closed forms of the definition they describe (gist.science
MegaFold technical summary, Methodik section 1 "EvoFlash-3D": exact softmax
attention whose logits carry an additively broadcast pair bias).  Logits are 0
and +-ln 3, so every softmax weight is 1/4 or 3/4 and every expected value below
is an exact rational number or a rational multiple of ln 3 / ln 4.  This script
calls neither the oracle nor the HIP library; it only writes the algebra out.
"""
import json
import math
import os

ln3 = math.log(3.0)
cases = {
    "_source": ("Hand-derived closed forms (no numeric example exists on the pages); "
                "written by make_hand_worked_n2.py, which calls no implementation."),
    "cases": [
        {
            "name": "bias_driven_q_zero",
            "derivation": [
                "R=1, N=2, H=1, d=1, q=0 so q.k/sqrt(d)=0 and the logits are the bias alone.",
                "bias[0,0,:]=[0, ln3] -> P[0,:]=[1/4,3/4]; bias[0,1,:]=[ln3, 0] -> P[1,:]=[3/4,1/4].",
                "v=[1,5]: O[0]=1/4+15/4=4, O[1]=3/4+5/4=2. lse[j]=ln(1+3)=ln 4 for both queries.",
                "dO=[1,1]: dP[j,k]=v[k]=[1,5]; D[0]=1/4+15/4=4, D[1]=3/4+5/4=2.",
                "dS[0,:]=[1/4(1-4), 3/4(5-4)]=[-3/4,3/4]; dS[1,:]=[3/4(1-2),1/4(5-2)]=[-3/4,3/4]; dBias=dS.",
                "dV[k]=sum_j P[j,k] dO[j]=[1,1]. k=[2,-1]: dQ[j]=sum_k dS[j,k] k[k]=-3/2-3/4=-9/4. dK=dS^T q=0.",
            ],
            "R": 1, "N": 2, "H": 1, "d": 1, "transpose": 0,
            "q": [[[[0.0]], [[0.0]]]], "k": [[[[2.0]], [[-1.0]]]], "v": [[[[1.0]], [[5.0]]]],
            "bias": [[[0.0, ln3], [ln3, 0.0]]], "mask": None, "dout": [[[[1.0]], [[1.0]]]],
            "expect": {
                "o": [[[[4.0]], [[2.0]]]], "lse": [[[math.log(4.0), math.log(4.0)]]],
                "dq": [[[[-2.25]], [[-2.25]]]], "dk": [[[[0.0]], [[0.0]]]],
                "dv": [[[[1.0]], [[1.0]]]], "dbias": [[[-0.75, 0.75], [-0.75, 0.75]]],
            },
        },
        {
            "name": "dot_product_driven",
            "derivation": [
                "R=1, N=2, H=1, d=4 so 1/sqrt(d)=1/2; no bias, no mask.",
                "k[0]=0, k[1]=e0; q[0]=2ln3 e0 -> logits [0, ln3] -> P[0,:]=[1/4,3/4];",
                "q[1]=-2ln3 e0 -> logits [0,-ln3] -> P[1,:]=[3/4,1/4]. lse[0]=ln 4, lse[1]=ln(4/3).",
                "v[0]=[1,2,0,0], v[1]=[5,-2,0,0]: O[0]=[4,-1,0,0], O[1]=[2,1,0,0].",
                "dO[0]=e0, dO[1]=e1: dP[0,:]=[1,5], D[0]=4; dP[1,:]=[2,-2], D[1]=3/2-1/2=1.",
                "dS[0,:]=[-3/4,3/4], dS[1,:]=[3/4,-3/4]; dBias=dS (one row).",
                "dQ[j]=sum_k dS[j,k]k[k]/2: dQ[0]=3/8 e0, dQ[1]=-3/8 e0.",
                "dK[k]=sum_j dS[j,k]q[j]/2: dK[0]=(-3/4*2ln3 + 3/4*(-2ln3))/2=-3/2 ln3, dK[1]=+3/2 ln3 (along e0).",
                "dV[k]=sum_j P[j,k]dO[j]: dV[0]=[1/4,3/4,0,0], dV[1]=[3/4,1/4,0,0].",
            ],
            "R": 1, "N": 2, "H": 1, "d": 4, "transpose": 0,
            "q": [[[[2 * ln3, 0, 0, 0]], [[-2 * ln3, 0, 0, 0]]]],
            "k": [[[[0.0, 0, 0, 0]], [[1.0, 0, 0, 0]]]],
            "v": [[[[1.0, 2.0, 0, 0]], [[5.0, -2.0, 0, 0]]]],
            "bias": None, "mask": None,
            "dout": [[[[1.0, 0, 0, 0]], [[0.0, 1.0, 0, 0]]]],
            "expect": {
                "o": [[[[4.0, -1.0, 0, 0]], [[2.0, 1.0, 0, 0]]]],
                "lse": [[[math.log(4.0), math.log(4.0 / 3.0)]]],
                "dq": [[[[0.375, 0, 0, 0]], [[-0.375, 0, 0, 0]]]],
                "dk": [[[[-1.5 * ln3, 0, 0, 0]], [[1.5 * ln3, 0, 0, 0]]]],
                "dv": [[[[0.25, 0.75, 0, 0]], [[0.75, 0.25, 0, 0]]]],
                "dbias": [[[-0.75, 0.75], [0.75, -0.75]]],
            },
        },
    ],
}

if __name__ == "__main__":
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hand_worked_n2.json")
    with open(out, "w") as f:
        json.dump(cases, f, indent=1)
