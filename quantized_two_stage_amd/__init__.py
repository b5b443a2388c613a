"""Two-stage quantized allreduce for MI355X (gfx950), W ranks simulated on one GPU.

``quantized_two_stage_amd.qr`` binds the C ABI of ``include/qr.h`` (built as
``libqr.so`` by ``quantized_two_stage_amd/build.py``); ``inputs`` holds the
seeded synthetic workloads.
"""
