"""The GPU tests' upload helpers (they live in ``workloads.device``, which the
benchmark uses as well)."""
from workloads.device import DevicePrep, DeviceWorkload, dev_f32, dev_i16, dev_i32, new_counters  # noqa: F401
