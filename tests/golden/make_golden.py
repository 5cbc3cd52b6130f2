"""Writes tests/golden/exact_small.json: small KDA cases evaluated in exact rational
arithmetic by ``oracle.exact`` (dense transition matrices, no rounding).

Run from the repository root:  python tests/golden/make_golden.py
Inputs are fixed rationals chosen by hand below (no randomness). Decays are
given as exact rationals; the fixture also stores log(alpha) as the float the
floating-point paths receive.
"""
import json
import math
import os
import sys
from fractions import Fraction as F

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle.exact import forward_exact  # noqa: E402


def case(name, q, k, v, alpha, beta, S0):
    o, S = forward_exact(q, k, v, alpha, beta, S0)
    return {
        "name": name,
        "inputs": {
            "q": [[str(x) for x in r] for r in q],
            "k": [[str(x) for x in r] for r in k],
            "v": [[str(x) for x in r] for r in v],
            "alpha": [[str(x) for x in r] for r in alpha],
            "log_alpha": [[math.log(x) for x in r] for r in alpha],
            "beta": [str(x) for x in beta],
            "initial_state": None if S0 is None else [[str(x) for x in r] for r in S0],
        },
        "expected": {
            "o": [[str(x) for x in r] for r in o],
            "final_state": [[str(x) for x in r] for r in S],
        },
    }


def main():
    h = F(1, 2)
    cases = [
        # dk = 3, dv = 2, zero initial state, mixed per-channel decays
        case("d3x2_zero_state",
             q=[[F(1), F(0), F(0)], [F(0), F(1), F(1)], [h, h, F(1)], [F(1), F(-1), F(0)]],
             k=[[F(0), F(1), F(0)], [F(1), F(0), F(0)], [F(2, 3), F(1, 3), F(2, 3)], [F(0), F(3, 5), F(4, 5)]],
             v=[[F(1), F(2)], [F(-1), F(1)], [F(3), F(0)], [F(1, 4), F(-2)]],
             alpha=[[F(1), F(1), F(1)], [h, F(3, 4), F(1)], [F(9, 10), h, F(1, 4)], [F(1), F(1, 8), F(7, 8)]],
             beta=[F(1), h, F(3, 4), F(1, 3)],
             S0=None),
        # dk = dv = 3, non-zero initial state, beta = 1 on a unit key (exact overwrite)
        case("d3x3_initial_state",
             q=[[F(1), F(1), F(0)], [F(0), F(0), F(1)], [F(1, 3), F(2, 3), F(2, 3)]],
             k=[[F(1), F(0), F(0)], [F(0), F(3, 5), F(4, 5)], [F(2, 3), F(2, 3), F(1, 3)]],
             v=[[F(2), F(-1), F(0)], [F(1), F(1), F(1)], [F(0), F(0), F(5)]],
             alpha=[[h, h, h], [F(1), F(1, 4), F(3, 4)], [F(2, 5), F(1), F(1, 10)]],
             beta=[F(1, 5), F(1), F(2, 3)],
             S0=[[F(1), F(2), F(0)], [F(0), F(-1), F(1)], [h, F(0), F(3)]]),
    ]
    out = {
        "description": "Exact rational KDA results from dense transition matrices (oracle.exact); "
                       "written by tests/golden/make_golden.py.",
        "citation": "GeekNews 'Kimi Linear' summary, section 'Kimi Delta Attention의 세밀한 메모리 제어' "
                    "(transition (I - beta k k^T) Diag(alpha)); 'From GPT-2 to Kimi K3' digest, sections "
                    "'DeltaNet -- 유한한 캐시의 덮어쓰기' and 'Kimi Linear (KDA) -- 채널별 세밀한 게이팅'.",
        "cases": cases,
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "exact_small.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1, ensure_ascii=False)
    print("wrote", path)


if __name__ == "__main__":
    main()
