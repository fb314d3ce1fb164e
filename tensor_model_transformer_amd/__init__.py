"""MI355X (gfx950) HIP implementation of one tensor-parallel rank's pre-LN
transformer layer shard, forward and backward, behind a C ABI
(``include/tp_layer.h``; library ``libtplayer.so`` built by ``build.py``).

Modules: ``binding`` (ctypes, argument marshalling only), ``shard`` (device
buffers via PyTorch), ``synth`` (seeded inputs), ``build`` (hipcc).
"""
