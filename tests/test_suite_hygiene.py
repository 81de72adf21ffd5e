"""The test suite itself: no module may define a top-level name twice.

Python keeps only the last definition of a repeated name, so a second copy
of a test function silently replaces the first and pytest never collects
it.  This parses every test module (no import, no GPU) and fails on any
repeated top-level function, class or assignment target.
"""
import ast
import glob
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def _top_level_names(tree):
    for node in tree.body:
        if isinstance(node, (ast.FunctionDef, ast.AsyncFunctionDef, ast.ClassDef)):
            yield node.name, node.lineno
        elif isinstance(node, ast.Assign):
            for t in node.targets:
                if isinstance(t, ast.Name):
                    yield t.id, node.lineno
        elif isinstance(node, ast.AnnAssign) and isinstance(node.target, ast.Name):
            yield node.target.id, node.lineno


def test_no_repeated_top_level_names_in_test_modules():
    problems = []
    files = sorted(glob.glob(os.path.join(HERE, "*.py")))
    assert files
    for path in files:
        with open(path) as f:
            tree = ast.parse(f.read(), filename=path)
        seen = {}
        for name, line in _top_level_names(tree):
            if name in seen:
                problems.append("%s: %s defined at lines %d and %d"
                                % (os.path.basename(path), name, seen[name], line))
            else:
                seen[name] = line
    assert not problems, "\n".join(problems)


def test_the_check_catches_a_repeated_test():
    src = "def test_a():\n    pass\n\nX = 1\n\ndef test_a():\n    pass\n"
    names = [n for n, _ in _top_level_names(ast.parse(src))]
    assert names.count("test_a") == 2
