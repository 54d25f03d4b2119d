"""Writes hand_example.txt from the closed form derived below (math only).

Problem (one sequence, one query head, one KV head, D = Dv = 2, sm_scale = 1,
k_scale = v_scale = 1, bf16-exact values):
  prefix keys   K0 = (1, 0), K1 = (0, 1);  values V0 = (1, 0), V1 = (0, 1)
  draft queries q0 = q1 = (1, 0)
  draft keys    k0 = (0, 0), k1 = (-1, 0); values v0 = (0, 0), v1 = (4, 4)
Row 0 sees K0, K1, k0 with scores 1, 0, 0 -> weights e, 1, 1:
  out0 = (e*V0 + V1 + v0) / (e + 2)
Row 1 additionally sees k1 with score -1 -> weight 1/e:
  out1 = (e*V0 + V1 + v0 + v1/e) / (e + 2 + 1/e)
"""
import math
import os

e = math.e
rows = [
    (e / (e + 2), 1 / (e + 2)),
    ((e + 4 / e) / (e + 2 + 1 / e), (1 + 4 / e) / (e + 2 + 1 / e)),
]
path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hand_example.txt")
with open(path, "w") as f:
    f.write("# closed-form output of the hand-worked example in make_hand_example.py\n")
    f.write("# one line per draft row, Dv = 2 values\n")
    for r in rows:
        f.write("%.17g %.17g\n" % r)
