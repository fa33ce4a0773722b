"""MI355X-native Differential Attention V2 forward pass (libdiffattn + thin binding)."""
__version__ = "0.1.0"
