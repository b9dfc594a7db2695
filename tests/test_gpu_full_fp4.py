"""Full-size parity, FP4 expert layer (DeepSeek-V4.1-Flash sizes): d=4096,
f=2880, 384 experts, top-6 renormalised, e2m1 with UE8M0 scales per 32
(17.93 MiB per expert), at 1, 16 and 1024 tokens on both expert paths and
with quantised activations.  Every token and every slot is compared with the
oracle: routing bit for bit, h within one bf16 step, out within the output
bars."""
import pytest

from full_size import FullSize

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def full():
    f = FullSize("fp4-e2m1").setup()
    yield f
    f.teardown()


@pytest.mark.parametrize("T,path", [(1, 0), (1, 2), (16, 0), (16, 2), (1024, 0)])
def test_fp4_e2m1(full, T, path):
    full.check(T, path)


@pytest.mark.parametrize("T", [16, 1024])
def test_fp4_e2m1_act_quant(full, T):
    full.check_act_quant(T)
