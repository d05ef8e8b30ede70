"""MI355X-native Test-Time-Training layer: a C-ABI HIP library (libttt.so) and
its thin Python binding (``linear_complexity_attention_amd.ttt``)."""

__all__ = ["ttt"]
