"""GPT-2 pre-norm decoder forward and cached decode on one MI355X (gfx950).

The compute path is the HIP library ``libgpt2mi.so`` built from ``csrc/``;
``gpt_pre_norm_amd.gpt2mi`` is its thin ctypes binding (argument marshalling
only).  Importing this package loads nothing; the binding loads the library on
first use and raises if it is missing.
"""
