"""MI355X-native GPT-2-style decoder-only forward pass behind a C ABI.

The compute lives in the HIP library built from `csrc/`; `lib` is its ctypes
binding and `synth` the seeded synthetic inputs.  Importing the package loads
nothing; `decoder_only_transformer_attn_amd.lib.load()` loads the library.
"""
