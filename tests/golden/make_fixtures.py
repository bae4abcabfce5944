"""Writes the hand-worked fixtures in this folder.

The expected values are closed forms derived by hand (the derivation is
stored in each fixture); nothing here calls the oracle or the HIP library.
Run from this folder: python make_fixtures.py
"""
import json
import math

ln2, ln3 = math.log(2.0), math.log(3.0)

refine = {
    "title": "Hand-worked linear attention and two-path refinement on a 1x3 token grid",
    "source": ("HSMLA full text (paperpeel), section 3.1 Z/D sums; section 3.3 "
               "local-neighbourhood, lin-local and two-path residual equations; "
               "window clipped to the grid (a reading)."),
    "shape": {"batch": 1, "grid_h": 1, "grid_w": 3, "heads": 1, "head_dim": 1,
              "block": 1, "window": 3},
    "qkv_layout": "per token [q, k, v]",
    "qkv": [[[1.0, 0.0, 6.0], [1.0, ln2, 12.0], [1.0, ln3, -6.0]]],
    "qkv_hat": [[[1.0, 1.0, 4.0], [2.0, 3.0, -4.0], [-1.0, -2.0, 100.0]]],
    "derivation": [
        "relu(k_hat) = [1, 3, 0]; Z = 1*4 + 3*(-4) + 0*100 = -8; D = 1 + 3 + 0 = 4.",
        "O_lin = Z/D = -2 for tokens 0 and 1 (q_hat > 0); token 2 has relu(q_hat) = 0, so 0/0 := 0.",
        "block 0 (token 0): window = tokens {0,1}; exp(q*k) = [1, 2]; O_local = (6 + 2*12)/3 = 10;",
        "  Z_W = -8, D_W = 4, lin-local = -2; O = -2 + 10 + 2 = 10.",
        "block 1 (token 1): window = {0,1,2}; exp(q*k) = [1,2,3]; O_local = (6 + 24 - 18)/6 = 2;",
        "  lin-local = -2; O = -2 + 2 + 2 = 2.",
        "block 2 (token 2): window = {1,2}; exp(q*k) = [2,3]; O_local = (24 - 18)/5 = 1.2;",
        "  relu(q_hat) = 0 so lin-local = 0; O = 0 + 1.2 - 0 = 1.2.",
        "selecting only block 1 leaves tokens 0 and 2 at O_lin: O = [-2, 2, 0].",
    ],
    "expected": {
        "Z": -8.0, "D": 4.0,
        "o_lin": [-2.0, -2.0, 0.0],
        "o_all_selected": [10.0, 2.0, 1.2],
        "o_select_block1": [-2.0, 2.0, 0.0],
    },
}

tok = []
for n in range(8):
    y, x = divmod(n, 4)
    blk = x // 2
    q0 = (4 * ln3 if n == 0 else 0.0) if blk == 0 else 0.0
    v1 = 0.0 if blk == 0 else -ln3
    tok.append([q0, 2.0, 5.0, -3.0, 11.0, v1])
gate = {
    "title": "Hand-worked block gate on a 2x4 token grid with 2x2 blocks, 2 heads of width 1",
    "source": ("HSMLA full text (paperpeel), section 3.2 head-level score and block-level "
               "aggregation (first equality: mean over heads of the sigmoids); mean-pooled "
               "block features."),
    "shape": {"batch": 1, "grid_h": 2, "grid_w": 4, "heads": 2, "head_dim": 1, "block": 2},
    "qkv_hat_layout": "per token [q_h0, q_h1, k_h0, k_h1, v_h0, v_h1]",
    "qkv_hat": [tok],
    "gate_w": [[1.0, 0.0, 0.0], [0.0, 0.0, 1.0]],
    "gate_w_layout": "per head [w_q, w_k, w_v]",
    "gate_b": [0.0, 0.0],
    "derivation": [
        "block 0 = tokens {0,1,4,5}; head 0 reads mean q_h0 = (4 ln3)/4 = ln3 -> sigmoid = 3/4;",
        "  head 1 reads mean v_h1 = 0 -> 1/2; M_0 = (3/4 + 1/2)/2 = 0.625.",
        "block 1 = tokens {2,3,6,7}; head 0: mean q_h0 = 0 -> 1/2; head 1: mean v_h1 = -ln3 -> 1/4;",
        "  M_1 = (1/2 + 1/4)/2 = 0.375.",
        "q_h1, k_h0, k_h1, v_h0 carry weight 0 and must not matter.",
        "a sigmoid of the mean logit would give sigmoid(ln3/2) = 0.634 for block 0 instead.",
        "top-1 selection: block 0.",
    ],
    "expected": {"scores": [0.625, 0.375], "top1": [0]},
}

if __name__ == "__main__":
    with open("refine_1x3.json", "w") as f:
        json.dump(refine, f, indent=1)
    with open("gate_2x4.json", "w") as f:
        json.dump(gate, f, indent=1)
