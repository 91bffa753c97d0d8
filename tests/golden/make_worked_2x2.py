"""Write ``worked_2x2.json``: a hand-worked 2x2 attention example in closed form.

The pages print no worked numbers, so this fixture evaluates closed forms
derived by hand (see each case's ``derivation``) with Python's ``math`` module
only. It calls neither the oracle nor the HIP library.

Q = [[1,2],[0,1]], K = [[1,0],[1,1]], V = [[1,2],[3,5]], scale = 0.5, hence
S = (Q K^T) * scale = [[0.5, 1.5], [0, 0.5]] (Q K^T is not symmetric, so a
transposed operand changes the result).
"""
import json
import math
import os


def main() -> None:
    e = math.e
    se = math.sqrt(e)
    V = [[1, 2], [3, 5]]

    def comb(w0, w1):
        return [w0 * V[0][c] + w1 * V[1][c] for c in range(2)]

    o0 = comb(1 / (1 + e), e / (1 + e))
    l0 = 0.5 + math.log(1 + e)
    o1 = comb(1 / (1 + se), se / (1 + se))
    l1 = math.log(1 + se)
    cases = [
        dict(name="full", causal=False, kv_len=2, q_start=0, O=[o0, o1], LSE=[l0, l1],
             derivation="row0 weights [1,e]/(1+e), LSE0=0.5+ln(1+e); "
                        "row1 weights [1,sqrt(e)]/(1+sqrt(e)), LSE1=ln(1+sqrt(e))"),
        dict(name="causal", causal=True, kv_len=2, q_start=0, O=[[1, 2], o1], LSE=[0.5, l1],
             derivation="row0 sees key0 only: O0=V0, LSE0=S00=0.5; row1 as in the full case"),
        dict(name="kv_len_1", causal=False, kv_len=1, q_start=0, O=[[1, 2], [1, 2]], LSE=[0.5, 0.0],
             derivation="only key0 valid: O=V0 for both rows, LSE_i=S_i0"),
        dict(name="q_start_1", causal=False, kv_len=2, q_start=1, O=[[0, 0], o1], LSE=[None, l1],
             derivation="row0 attends to nothing: O0=0, LSE0=-inf (stored as null); row1 as in the full case"),
    ]
    fx = dict(
        about="Hand-worked 2x2 example of softmax(Q K^T * scale + mask) V with closed-form results.",
        cites=[
            "aiknowledge.cn '4.5 注意力优化实战：从PyTorch到CUDA的完整流程', step 1 baseline implementation: "
            "scores Q K^T times scale, masked entries set to -inf, softmax over keys, weighted sum of V",
            "Profiling in PyTorch (part 3): the causal mask is the lower triangle; the math backend's safe "
            "softmax gives 0 for a row whose entries are all -inf",
        ],
        Q=[[1, 2], [0, 1]], K=[[1, 0], [1, 1]], V=V, scale=0.5, cases=cases)
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "worked_2x2.json")
    with open(path, "w", encoding="utf-8") as f:
        json.dump(fx, f, indent=1, ensure_ascii=False)
        f.write("\n")


if __name__ == "__main__":
    main()
