"""Shared helpers for the GPU tests: the seeded device setup (``workload``) and the
parity bar (``oracle.compare``), re-exported under one name."""
from oracle.compare import NEAR_TIE, parity, same_set  # noqa: F401
from workload import HostLayer  # noqa: F401
from workload.device_layer import DeviceCanonicalLayer, DeviceLayer, config_for  # noqa: F401
