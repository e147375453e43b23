"""CPU oracle for the SVDQuant linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link anything in this package; only the tests, the smoke check of the entry
module and the CPU-baseline leg of the benchmark use it.  It shares no code
with the HIP library: the two meet only through the seeded inputs of
``diffusion_smooth_group_amd.workloads``, which hold no arithmetic of the
method.

It is a plain, slow, float64 restatement of the method as the SVDQuant paper
describes it ("SVDQuant: Absorbing Outliers by Low-Rank Components for 4-Bit
Diffusion Models", read in the translated article on developer.volcengine.com;
cited below as [SVDQuant §n]).
"""
from .svdquant import *  # noqa: F401,F403
