"""Whether the GPU tests can run here, and what happens when they cannot.

A GPU test module calls ``need_gpu()`` before anything else touches the
device.  Without a usable GPU (torch missing, no device visible to torch, or
the HIP library not built) the module is skipped -- unless GPU use is
required, in which case the module errors instead, so that a suite run on a
box whose runtime failed to come up cannot pass having run nothing.  GPU use
is required when ``PGQA_REQUIRE_GPU=1``, and by default on a machine that has
the GPU driver's device node (/dev/kfd); ``PGQA_REQUIRE_GPU=0`` turns it off.
"""
import os

import pytest


def gpu_required() -> bool:
    flag = os.environ.get("PGQA_REQUIRE_GPU")
    if flag is not None and flag != "":
        return flag == "1"
    return os.path.exists("/dev/kfd")


def why_no_gpu():
    """None if the GPU tests can run, else the reason they cannot."""
    try:
        import torch
    except ImportError as e:
        return f"torch is not importable ({e})"
    if not torch.cuda.is_available():
        return "no GPU visible to torch"
    try:
        import paged_gqa_decode_attn_amd as pg
        pg.lib()
    except Exception as e:  # missing or unloadable HIP library
        return f"the HIP library did not load ({e})"
    return None


def need_gpu():
    reason = why_no_gpu()
    if reason is None:
        return
    if gpu_required():
        pytest.fail(f"GPU tests required (PGQA_REQUIRE_GPU / /dev/kfd) but {reason}", pytrace=False)
    pytest.skip(f"needs a GPU: {reason}", allow_module_level=True)
