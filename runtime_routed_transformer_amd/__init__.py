"""Library-of-Layers routed-core forward pass on AMD MI355X (gfx950).

Modules:
  workloads  seeded synthetic inputs of the five workloads (no method arithmetic)
  binding    ctypes binding of liblol_core (include/lol_core.h), same names
  core       device-resident inputs + a forward call through the binding
  build_lib  builds lib/liblol_core.so from csrc/*.hip with hipcc
"""
from . import workloads  # noqa: F401

__all__ = ["workloads", "binding", "core", "build_lib"]
