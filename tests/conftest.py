import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# The schedule, scoring-path and key-split tests pin the library's choices
# through its debug overrides, which it reads only while FWPKM_DEBUG is "1".
os.environ["FWPKM_DEBUG"] = "1"
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: larger CPU cases")
