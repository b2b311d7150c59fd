"""Host side of the GPU pattern search (CPU only: no kernel is launched).

The search's arithmetic (work counts and recall) runs in the library; what is
left on the host is the choice among candidates, checked here on hand-made
tables, and the rule that the module does no arithmetic of the method itself.
"""
import os
import re

from dynamic_sparse_attention_index_amd import pattern_search as PS


def test_choice_rule_on_hand_made_tables():
    blocks = [[10, 20, 30], [10, 20, 30], [10, 20, 30], [10, 20, 30]]
    recall = [[0.5, 0.9, 0.95],   # best recall within budget 25 is candidate 1
              [0.9, 0.9, 0.95],   # equal recall: the lower work wins
              [0.9, 0.8, 0.99],   # budget 30 admits candidate 2
              [0.9, 0.9, 0.9]]    # nothing fits budget 5
    assert PS.choose(blocks, recall, [25, 25, 30, 5]) == [1, 0, 2, -1]
    # equal recall and equal work: the earlier candidate
    assert PS.choose([[5, 5]], [[0.7, 0.7]], [10]) == [0]


def test_module_does_no_method_arithmetic():
    src = open(os.path.join(os.path.dirname(PS.__file__), "pattern_search.py")).read()
    code = "\n".join(line.split("#")[0] for line in src.splitlines())
    for pat in (r"torch\.(exp|log|cumsum|sum|mean|where|clamp|maximum|minimum|isneginf)\b",
                r"\.(exp|cumsum|sum|mean)\(", r"torch\.split"):
        assert not re.search(pat, code), pat
