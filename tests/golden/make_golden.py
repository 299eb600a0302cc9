"""Write the hand-derived worked examples in this folder.

The pages print no worked example, so these fixtures are small cases whose
outputs follow in closed form from the recurrence itself (exponential-Euler
discretisation, "Efficient Sequence Modeling: From S4 to Mamba-3", sections 03
and 04; selective SSM of Gu & Dao 2023, cited by the ssm-bench README).
Each expected value is derived in the ``derivation`` field and computed here
from that formula with ``math`` only -- no oracle, no GPU.
"""
import json
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LN2, LN3 = math.log(2.0), math.log(3.0)


def impulse_mamba1():
    # channel 0: Delta = 1, A = [-ln2, -ln4] -> Abar = [1/2, 1/4]; x = impulse 1
    # channel 1: Delta = 1/2, A = [-2ln2, -4ln2] -> Abar = [1/2, 1/4]; x = impulse 2
    # B_t = C_t = [1, 1]; h0 = 0; D = [0, 1]; no gate.
    L = 4
    y0 = [0.5 ** t + 0.25 ** t for t in range(L)]
    y1 = [v + (2.0 if t == 0 else 0.0) for t, v in enumerate(y0)]
    return dict(
        name="mamba1_impulse",
        cite="recurrence h_t = exp(Delta_t A) h_{t-1} + Delta_t B_t x_t, y_t = C_t.h_t + D x_t "
             "(Gu & Dao 2023; exponential-Euler, S4-to-Mamba-3 case study sec. 04)",
        derivation="Delta_0 x_0 B_0 = 1 in both channels, so h_t[n] = Abar_n^t and "
                   "y_t = 2^-t + 4^-t (+ D x_t = 2 at t=0 in channel 1); h_final = [1/8, 1/64].",
        inputs=dict(
            x=[[[1.0, 2.0], [0.0, 0.0], [0.0, 0.0], [0.0, 0.0]]],
            delta=[[[1.0, 0.5] for _ in range(L)]],
            A=[[-LN2, -2 * LN2], [-2 * LN2, -4 * LN2]],
            Bm=[[[1.0, 1.0] for _ in range(L)]],
            Cm=[[[1.0, 1.0] for _ in range(L)]],
            D=[0.0, 1.0], z=None, h0=None),
        expected=dict(
            y=[[[y0[t], y1[t]] for t in range(L)]],
            h_final=[[[0.125, 1.0 / 64], [0.125, 1.0 / 64]]]),
    )


def gated_step():
    # state 2, A = -1, Delta = ln2 -> Abar = 1/2; B = 1, x = 1 -> h = 1 + ln2
    # C = 2, D = 1/2, z = ln3 -> sigmoid(z) = 3/4, silu(z) = (3/4) ln3
    h = 1.0 + LN2
    y = (2.0 * h + 0.5) * 0.75 * LN3
    return dict(
        name="gated_step",
        cite="one decode step of the same recurrence with the silu(z) gate "
             "(S4-to-Mamba-3 case study sec. 03: incremental step())",
        derivation="h = (1/2)*2 + ln2*1*1 = 1 + ln2; y = (C h + D x) * z*sigmoid(z) "
                   "= (2(1+ln2) + 1/2) * (3/4) ln3.",
        inputs=dict(state=[[[2.0]]], x=[[1.0]], delta=[[LN2]], A=[[-1.0]], Bm=[[1.0]],
                    Cm=[[2.0]], D=[0.5], z=[[LN3]]),
        expected=dict(y=[[y]], state=[[[h]]]),
    )


def ssd_carry():
    # H = 1, P = 2, N = 1, L = 4; A_h = -ln2, Delta = 1 -> a = 1/2; B = C = 1
    # x = impulse [1, 2] at t = 0; h0 = [[1, -1]]
    # S_t[p] = (1/2)^{t+1} h0[p] + (1/2)^t x_0[p]; y_t[p] = S_t[p]
    L = 4
    S = [[0.5 ** (t + 1) * h + 0.5 ** t * x for h, x in zip([1.0, -1.0], [1.0, 2.0])]
         for t in range(L)]
    return dict(
        name="ssd_carry",
        cite="SSD with scalar decay per head and (N,P) state carried across chunks "
             "(S4-to-Mamba-3 case study sec. 03 mamba2_minimal.py, sec. 04)",
        derivation="S_t[p] = 2^-(t+1) h0[p] + 2^-t x_0[p] = [1.5, 1.5], [.75, .75], "
                   "[.375, .375], [.1875, .1875]; the chunked form must carry the state "
                   "across every chunk boundary (chunks 1, 2, 3 and 4).",
        inputs=dict(x=[[[[1.0, 2.0]], [[0.0, 0.0]], [[0.0, 0.0]], [[0.0, 0.0]]]],
                    delta=[[[1.0] for _ in range(L)]], A=[-LN2],
                    Bm=[[[1.0] for _ in range(L)]], Cm=[[[1.0] for _ in range(L)]],
                    D=None, z=None, h0=[[[[1.0, -1.0]]]]),
        expected=dict(y=[[[S[t]] for t in range(L)]], h_final=[[[S[-1]]]]),
        chunks=[1, 2, 3, 4, 8],
    )


if __name__ == "__main__":
    for fx in (impulse_mamba1(), gated_step(), ssd_carry()):
        with open(os.path.join(HERE, fx["name"] + ".json"), "w") as f:
            json.dump(fx, f, indent=1)
        print("wrote", fx["name"])
