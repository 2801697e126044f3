"""Write tests/golden/one_token_softmax.json: a hand-built one-token example and the oracle's
output on it.  Calls only oracle/.

The pages print no worked numerical example, so the example is built by hand to make every
quantity a closed form: d = 2, E = 3, f = 1, x = [1, 2].  W_r's columns give logits
[1, 0, 1] (a tie between experts 0 and 2, which the lower index wins).  The experts give
y0 = [2 SiLU(1), 0], y1 = [0, SiLU(2)], y2 = -SiLU(3) [1, 1]; the shared expert gives
SiLU(2) [1, 1].  tests/test_oracle_ffn.py checks the stored oracle outputs against those
closed forms.  Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
import oracle  # noqa: E402

EX = {
    "about": "one-token softmax example; logical layouts W_r [d,E], gate/up [d,f], down [f,d]",
    "x": [1.0, 2.0],
    "w_router": [[1.0, 0.0, 1.0], [0.0, 0.0, 0.0]],
    "experts": [
        {"gate": [[1.0], [0.0]], "up": [[0.0], [1.0]], "down": [[1.0, 0.0]]},
        {"gate": [[0.0], [1.0]], "up": [[1.0], [0.0]], "down": [[0.0, 1.0]]},
        {"gate": [[1.0], [1.0]], "up": [[1.0], [-1.0]], "down": [[1.0, 1.0]]},
    ],
    "shared": {"gate": [[0.0], [1.0]], "up": [[1.0], [0.0]], "down": [[1.0, 1.0]]},
}


def main():
    f32 = lambda a: np.array(a, np.float32)  # noqa: E731
    x = np.array([EX["x"]])
    l = oracle.router_logits(x, f32(EX["w_router"]))
    routed = oracle.ExpertSet(3, [f32(e["gate"]) for e in EX["experts"]],
                              [f32(e["up"]) for e in EX["experts"]],
                              [f32(e["down"]) for e in EX["experts"]])
    sh = EX["shared"]
    shared = oracle.ExpertSet(1, [f32(sh["gate"])], [f32(sh["up"])], [f32(sh["down"])])
    out = {}
    for k in (1, 2, 3):
        ids, w, _ = oracle.route(l, k)
        out[str(k)] = oracle.moe_tokens(x, ids, w, routed, shared, 2, 1, 1)[0].tolist()
    doc = dict(EX, oracle_out=out)
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "one_token_softmax.json")
    with open(path, "w") as fh:
        json.dump(doc, fh, indent=1)
        fh.write("\n")
    print(path)


if __name__ == "__main__":
    main()
