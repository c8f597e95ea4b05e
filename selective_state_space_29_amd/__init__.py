"""MI355X-native Mamba selective-scan forward: a C-ABI HIP library plus a thin Python binding.

``selective_scan_fn`` (in :mod:`.scan`) is the user entry point; :mod:`.gen` and
:mod:`.workloads` provide the seeded synthetic inputs.
"""

__all__ = ["selective_scan_fn"]


def __getattr__(name):
    if name == "selective_scan_fn":
        from .scan import selective_scan_fn

        return selective_scan_fn
    raise AttributeError(name)
