"""Parsers for the hand-worked fixtures in this folder (each fixture cites its source)."""
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def read_cases(name: str) -> list:
    """Parse 'case <name> ... end' blocks of 'key values...' lines; '#' starts a comment."""
    cases, cur = [], None
    with open(os.path.join(HERE, name)) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            key, _, rest = line.partition(" ")
            if key == "case":
                cur = {"name": rest.strip(), "q": []}
            elif key == "end":
                cases.append(cur)
                cur = None
            elif key == "q":
                cur["q"].append([float(x) for x in rest.split()])
            else:
                cur[key] = rest.split()
    return cases


def parse_paths(tokens: list) -> list:
    return [tuple(int(t) for t in p.split(".")) for p in tokens]
