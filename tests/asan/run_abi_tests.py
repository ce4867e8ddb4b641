"""Run tests/test_abi.py against another build of the library (the
sanitizer build): python run_abi_tests.py LIB.so"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))
import block_scaled_quantized_qgemm_amd._lib as L  # noqa: E402

L.LIB_PATH = os.path.abspath(sys.argv[1])
import pytest  # noqa: E402

sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", os.path.join(ROOT, "tests", "test_abi.py")]))
