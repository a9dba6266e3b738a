"""The oracle and the HIP path share no code: neither imports the other, and
the product package never touches the oracle (static check of the sources)."""
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _sources(d, exts):
    for dp, _, fs in os.walk(os.path.join(ROOT, d)):
        for f in fs:
            if f.endswith(exts):
                yield os.path.join(dp, f)


def test_oracle_does_not_import_product():
    for p in _sources("oracle", (".py", ".c", ".h")):
        s = open(p).read()
        assert "chunked_kl_loss_02_amd" not in s, p
        assert "kdkl" not in s, p


def test_product_does_not_import_oracle():
    pat = re.compile(r"^\s*(from|import)\s+oracle\b", re.M)
    for p in _sources("chunked_kl_loss_02_amd", (".py", ".hip", ".cpp", ".h", ".hpp")):
        s = open(p).read()
        assert not pat.search(s), p
        assert "oracle" not in s.lower(), p
