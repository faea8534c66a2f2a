"""Writes closed_forms.json: small attention problems whose answers follow by
hand from the formulas on the reference pages. Uses only the math module (no
oracle, no GPU code), so the stored values pin the oracle from outside.

Run: python tests/golden/make_golden.py
"""
import json
import math
import os

E = math.e
cases = []

# 1. Two keys, no mask. S = [1, 0]; softmax = [e, 1]/(e+1); O = sum p_j v_j;
#    lse = log(e + 1).  CANN flash_attn page: attention and softmax_lse formulas.
p0, p1 = E / (E + 1), 1 / (E + 1)
cases.append(dict(
    name="two_keys", cite="CANN flash_attn: attention formula; softmax_lse formula",
    kind="rows", q=[[1.0, 0.0]], k=[[1.0, 0.0], [0.0, 1.0]], v=[[1.0, 2.0], [3.0, 4.0]],
    scale=1.0, o=[[p0 * 1 + p1 * 3, p0 * 2 + p1 * 4]], lse=[math.log(E + 1)]))

# 2. Same with scale 1/2 and q doubled: identical scores, identical answer.
cases.append(dict(
    name="scale_applied_to_scores", cite="CANN flash_attn: S = QK^T / sqrt(d) (scale on QK^T)",
    kind="rows", q=[[2.0, 0.0]], k=[[1.0, 0.0], [0.0, 1.0]], v=[[1.0, 2.0], [3.0, 4.0]],
    scale=0.5, o=[[p0 * 1 + p1 * 3, p0 * 2 + p1 * 4]], lse=[math.log(E + 1)]))

# 3. Sink 0.5 on case 1: m = max(0.5, 1) = 1; denominator e^0 + e^-1 + e^-0.5;
#    numerator e^0 v_0 + e^-1 v_1. lse keeps max(S) only (sink-free).
den = 1 + math.exp(-1) + math.exp(-0.5)
cases.append(dict(
    name="two_keys_sink", cite="CANN flash_attn: sink formulas m = max(sink, max S); softmax_lse formula",
    kind="rows", q=[[1.0, 0.0]], k=[[1.0, 0.0], [0.0, 1.0]], v=[[1.0, 2.0], [3.0, 4.0]],
    scale=1.0, sink=0.5,
    o=[[(1 + 3 * math.exp(-1)) / den, (2 + 4 * math.exp(-1)) / den]], lse=[math.log(E + 1)]))

# 4. Bottom-right causal with Lq=2, Lk=4, all scores 0: query 0 sees keys
#    0..2, query 1 sees 0..3; O = mean of visible values, lse = log(count).
cases.append(dict(
    name="causal_bottom_right", cite="MindSpore sparse_flash_attention: sparse_mode 3 rightDownCausal",
    kind="dense", q=[[[[0.0]], [[0.0]]]], k=[[[[1.0]], [[2.0]], [[3.0]], [[4.0]]]],
    v=[[[[1.0]], [[2.0]], [[3.0]], [[4.0]]]], scale=1.0, causal=True, window=[-1, -1],
    o=[[[[2.0]], [[2.5]]]], lse=[[[math.log(3), math.log(4)]]]))

# 5. Sliding window (left=1, right=0) on Lq=Lk=5, scores 0, v_j = j:
#    query t sees {t-1, t}.  lite_boost flash_attention: window_size argument.
cases.append(dict(
    name="window_left1_right0", cite="lite_boost flash_attention: window_size (left, right)",
    kind="dense", q=[[[[0.0]]] * 5], k=[[[[0.0]]] * 5], v=[[[[float(j)]] for j in range(5)]],
    scale=1.0, causal=False, window=[1, 0],
    o=[[[[0.0]], [[0.5]], [[1.5]], [[2.5]], [[3.5]]]],
    lse=[[[0.0] + [math.log(2)] * 4]]))

# 6. Window (left=0, right=1), non-causal: query t sees {t, t+1}.
cases.append(dict(
    name="window_left0_right1", cite="lite_boost flash_attention: window_size (left, right)",
    kind="dense", q=[[[[0.0]]] * 5], k=[[[[0.0]]] * 5], v=[[[[float(j)]] for j in range(5)]],
    scale=1.0, causal=False, window=[0, 1],
    o=[[[[0.5]], [[1.5]], [[2.5]], [[3.5]], [[4.0]]]],
    lse=[[[math.log(2)] * 4 + [0.0]]]))

# 7. GQA, Hq=4, Hkv=2: heads 0,1 read KV head 0 and heads 2,3 read KV head 1.
#    KV head 0 has keys e0,e1 with values 1,0; KV head 1 has keys e0,e1 with
#    values 0,1. q for every head is e0, so S = [1, 0] for all heads:
#    heads 0,1 give O = e/(e+1); heads 2,3 give O = 1/(e+1).
#    MindSpore sparse_flash_attention: softmax_max shape (B, N2, S1, N1/N2).
cases.append(dict(
    name="gqa_grouping", cite="MindSpore sparse_flash_attention: grouping (N2, N1/N2)",
    kind="dense", q=[[[[1.0, 0.0]] * 4]],
    k=[[[[1.0, 0.0], [1.0, 0.0]], [[0.0, 1.0], [0.0, 1.0]]]],
    v=[[[[1.0], [0.0]], [[0.0], [1.0]]]], scale=1.0, causal=False, window=[-1, -1],
    o=[[[[p0], [p0], [p1], [p1]]]], lse=[[[math.log(E + 1)]] * 4]))

# 8. Combine two split results with LSE log 2 and log 3: weights 2/5, 3/5,
#    merged LSE log 5. With sink log 5 the denominator gains exp(0) = 1 when
#    measured against M* = log 5: weights 0.4, 0.6 over 2.0.
#    MATE flash_attn_combine; CANN softmax_lse (ring-attention merge).
cases.append(dict(
    name="combine_two_splits", cite="MATE flash_attn_combine; CANN softmax_lse formula",
    kind="combine", o_partial=[[[1.0, 0.0]], [[0.0, 1.0]]], lse_partial=[[math.log(2)], [math.log(3)]],
    o=[0.4, 0.6], lse=math.log(5), sink=math.log(5), o_sink=[0.2, 0.3]))

# 9. Sparse indices [0, 0, 1, -1, 7] against Sk = 4, all scores 0, v_j = j:
#    -1 and 7 are skipped, key 0 counts twice: O = (0+0+1)/3, lse = log 3.
cases.append(dict(
    name="sparse_duplicates_and_padding",
    cite="MindSpore sparse_flash_attention: sparse_indices select K~, V~",
    kind="sparse", sq=1, sk=4, indices=[0, 0, 1, -1, 7], mode=0,
    o=1.0 / 3.0, lse=math.log(3)))

path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "closed_forms.json")
with open(path, "w") as f:
    json.dump(cases, f, indent=1)
print("wrote", path, len(cases), "cases")
