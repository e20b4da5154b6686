"""Write rope_d2_worked_example.json: a T=3, D=2 attention worked out in closed form.

The pages print no attention values, so this fixture is derived by hand from the
definition (not from the oracle and not from the HIP path):
  * D = 2 has one rotary pair with theta_0 = base^0 = 1, so position t rotates the
    pair (x0, x1), read as the complex number x0 + i x1, by e^{i t}, for any base.
  * score(i, j) = Re(conj(q_i e^{i i}) k_j e^{i j}) / sqrt(2)
               = Re(conj(q_i) k_j e^{i (j - i)}) / sqrt(2),  j <= i.
  * lse_i = log sum_{j<=i} exp(score(i, j));  o_i = sum_j exp(score(i, j) - lse_i) v_j.
"""
import cmath
import json
import math
import os

q = [(1.0, 0.0), (0.0, 1.0), (1.0, 1.0)]
k = [(1.0, 0.0), (1.0, -1.0), (0.0, 2.0)]
v = [(1.0, 2.0), (3.0, -1.0), (-2.0, 0.5)]
base = 10000.0


def main():
    lse, o = [], []
    for i in range(3):
        qi = complex(*q[i])
        s = [(qi.conjugate() * complex(*k[j]) * cmath.exp(1j * (j - i))).real / math.sqrt(2)
             for j in range(i + 1)]
        z = math.fsum(math.exp(x) for x in s)
        lse.append(math.log(z))
        o.append([math.fsum(math.exp(s[j]) * v[j][d] for j in range(i + 1)) / z for d in range(2)])
    out = {
        "source": "closed form for D=2 (theta_0 = 1); see make_d2_worked_example.py",
        "rope_base": base, "q": q, "k": k, "v": v, "lse": lse, "o": o,
    }
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "rope_d2_worked_example.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
