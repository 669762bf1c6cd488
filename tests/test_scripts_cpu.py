"""The GPU-only scripts (bench.py, the smoke check) cannot run on a CPU
host; at least every global name their functions read must exist at module
level, so a renamed variable fails here rather than on the GPU."""
import builtins
import os
import symtable

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MODULE_DUNDERS = {"__file__", "__name__", "__doc__", "__spec__", "__package__"}


def undefined_globals(path):
    src = open(path).read()
    top = symtable.symtable(src, path, "exec")
    defined = {s.get_name() for s in top.get_symbols() if s.is_assigned() or s.is_imported()}
    missing = []

    def walk(table):
        for child in table.get_children():
            for s in child.get_symbols():
                name = s.get_name()
                if (s.is_referenced() and s.is_global() and name not in defined
                        and name not in MODULE_DUNDERS and not hasattr(builtins, name)):
                    missing.append((child.get_name(), name))
            walk(child)

    walk(top)
    return missing


@pytest.mark.parametrize("rel", ["bench.py", "__graft_entry__.py", "state_memory_attention_amd/dart.py",
                                 "state_memory_attention_amd/synth.py", "state_memory_attention_amd/build.py"])
def test_no_undefined_global_names(rel):
    assert undefined_globals(os.path.join(ROOT, rel)) == []


def test_the_check_finds_an_undefined_name(tmp_path):
    p = tmp_path / "m.py"
    p.write_text("import os\nX = 1\n\ndef f():\n    return os.sep, X, len, y_missing\n")
    assert undefined_globals(str(p)) == [("f", "y_missing")]
