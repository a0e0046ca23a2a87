"""libzeroshard for AMD Instinct MI355X: the per-rank ZeRO-2 optimizer-shard step.

  zeroshard  -- ctypes binding of the C ABI (include/zeroshard.h); importing it
                loads libzeroshard.so and raises if it is not built.
  synth      -- seeded synthetic inputs (host and device twins) and the
                workload definitions used by the tests and the benchmark.
  build      -- compiles the in-tree shared libraries.
"""
__all__ = ["zeroshard", "synth", "build"]
