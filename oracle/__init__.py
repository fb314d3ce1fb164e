"""fp64 CPU oracle of the tensor-parallel layer shard.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product path, and
it shares no code with the HIP path.

Modules:
  layer  -- the layer definition in NumPy fp64 (LOCAL, FULL, PARTIALS modes)
  brute  -- pure-Python loop forward of the same layer (independent pin)
  fd     -- central finite differences of loss = sum(out * dout)
  decode -- one decode step against a per-rank KV cache shard
"""
