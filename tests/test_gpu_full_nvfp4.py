"""Full-size parity, NVFP4 expert layer: the FP4 layer's shape (d=4096,
f=2880, 384 experts, top-6 renormalised) with e2m1 codes and one e4m3 scale
per 16 inputs (19.9 MB per expert), at 1, 16 and 1024 tokens on both expert
paths.  Every token and every slot is compared with the oracle: routing bit
for bit, h within one bf16 step, out within the output bars."""
import pytest

from full_size import FullSize

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def full():
    f = FullSize("fp4-nvfp4").setup()
    yield f
    f.teardown()


@pytest.mark.parametrize("T,path", [(1, 0), (16, 0), (16, 2), (1024, 0), (1024, 1)])
def test_fp4_nvfp4(full, T, path):
    full.check(T, path)
