"""Readers for the hand-written fixtures under tests/golden/."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                yield line.split()


def indexer_hand():
    d = {"k": {}, "q": {}, "w": {}, "I": {}, "topk": []}
    for tok in _lines("indexer_hand.txt"):
        key = tok[0]
        if key in ("HI", "dI"):
            d[key] = int(tok[1])
        elif key == "k":
            d["k"][int(tok[1])] = ([int(c, 16) for c in tok[2:-2]], float(tok[-1]))
        elif key == "q":
            d["q"][(int(tok[1]), int(tok[2]))] = ([int(c, 16) for c in tok[3:-2]], float(tok[-1]))
        elif key == "w":
            d["w"][int(tok[1])] = [float(x) for x in tok[2:]]
        elif key == "I":
            d["I"][(int(tok[1]), int(tok[2]))] = float(tok[3])
        elif key == "topk":
            d["topk"].append((int(tok[1]), int(tok[2]), [int(x) for x in tok[3:]]))
    return d


def topk_ties():
    scores, cases = None, []
    for tok in _lines("topk_ties.txt"):
        if tok[0] == "scores":
            scores = [float(x) for x in tok[1:]]
        elif tok[0] == "case":
            cases.append((int(tok[1]), [int(x) for x in tok[2:]]))
    return scores, cases
