"""CPU oracle package -- test infrastructure only (tests/, smoke(), bench cpu_baseline)."""
from .moeq8_ref import *  # noqa: F401,F403
