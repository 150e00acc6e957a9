"""Write t0_handworked.json: a hand-worked MSA decode example.

Structure from the diagram described in "MiniMax wird dünn: M3-Attention
anhand eines einzigen Diagramms entschlüsselt" (atlascloud.ai), section 1,
"Schritt 1: Index-Branch" and "Schritt 2: Sparse-Branch": six query heads in
two GQA groups, one index query per group, one shared index-key head; heads
Q1-Q3 use index list I_1 and Q4-Q6 use I_2.

Every expected value below is derived by hand from the inputs (the working is
in the "derivation" strings) and evaluated here from its closed form; nothing
is computed by the oracle or the GPU path.
"""
import json
import math
import os

e = math.e
# tokens 0..6, block size 2 -> blocks {0,1} {2,3} {4,5} {6}; current token 6,
# own block c = (7-1)//2 = 3; eligible blocks 0, 1, 2; k = 2 -> one chosen + own.
case = {
    "citation": "MiniMax wird dünn (atlascloud.ai), section 1, Schritt 1 and Schritt 2: "
                "6 heads, 2 groups, one index query per group, single-head index key, "
                "block max pool, top-k; Q1-Q3 use I_1, Q4-Q6 use I_2",
    "shape": {"num_q_heads": 6, "num_kv_heads": 2, "head_dim": 2, "num_idx_heads": 1,
              "idx_dim": 2, "block_size": 2, "top_k": 2},
    "softmax_scale": 1.0,
    "seq_len": 7,
    "idx_q": [[[1, 0]], [[0, 1]]],
    "idx_k": [[1, 3], [2, 0], [4, 1], [0, 0], [3, 2], [-1, 5], [9, 9]],
    # keys/values per group, per token [L][D]; unselected tokens carry values
    # that would change the answer if they were used
    "k": [[[0, 0]] * 7,
          [[5, 5], [5, 5], [5, 5], [5, 5], [1, 0], [0, 0], [2, 0]]],
    "v": [[[t, 10 * t] for t in range(7)],
          [[100, 100], [100, 100], [100, 100], [100, 100], [1, 0], [0, 1], [1, 1]]],
    "q": [[0, 0], [1, -1], [2, -2], [1, 0], [0, 0], [2, 0]],
    "derivation": [
        "group 0 index query [1,0]: token scores 1,2 | 4,0 | 3,-1 -> pooled [2,4,3]",
        "group 1 index query [0,1]: token scores 3,0 | 1,0 | 2,5 -> pooled [3,1,5]",
        "k=2 keeps the best eligible block plus own block 3: I_1=[1,3], I_2=[2,3]",
        "heads 0-2: group-0 keys are zero, weights uniform over tokens 2,3,6: "
        "out = ([2,20]+[3,30]+[6,60])/3 = [11/3, 110/3]",
        "head 3: q=[1,0], tokens 4,5,6 scores 1,0,2: out = [(e+e^2), (1+e^2)]/(e+1+e^2)",
        "head 4: q=[0,0], uniform over tokens 4,5,6: out = [2/3, 2/3]",
        "head 5: q=[2,0], scores 2,0,4: out = [(e^2+e^4), (1+e^4)]/(e^2+1+e^4)",
    ],
    "expected_pooled": [[2, 4, 3], [3, 1, 5]],
    "expected_sel": [[1, 3], [2, 3]],
    "expected_out": [
        [11 / 3, 110 / 3], [11 / 3, 110 / 3], [11 / 3, 110 / 3],
        [(e + e**2) / (e + 1 + e**2), (1 + e**2) / (e + 1 + e**2)],
        [2 / 3, 2 / 3],
        [(e**2 + e**4) / (e**2 + 1 + e**4), (1 + e**4) / (e**2 + 1 + e**4)],
    ],
}

if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "t0_handworked.json")
    with open(path, "w") as f:
        json.dump(case, f, indent=1)
    print("wrote", path)
