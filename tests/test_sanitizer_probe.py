"""Run inside the sanitizer children of tests/test_sanitizers.py: the build
under test is the one actually loaded (a plain run checks nothing here)."""
import os


def test_the_selected_builds_are_loaded():
    lib = os.environ.get("KDA_LIBRARY")
    if lib:
        from gated_delta_rule_101_amd import kda
        assert kda.load_library()._name == lib
    olib = os.environ.get("KDA_ORACLE_LIBRARY")
    if olib:
        from oracle import default
        assert default().path == olib
