"""MI355X (gfx950) library for the CPR-scheduled gated delta-rule layer.

The compute path is the HIP shared library under csrc/ (C ABI, include/gdn.h);
`binding` marshals torch tensors into it.  Importing this package loads
nothing; `binding.lib()` loads the library and raises if it is not built.
"""
