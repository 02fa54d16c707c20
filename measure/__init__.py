"""Measurement tools beside bench.py: the streaming-bandwidth probe and the
rocprofv3 summariser whose outputs profiles/ keeps.  Not part of the library."""
