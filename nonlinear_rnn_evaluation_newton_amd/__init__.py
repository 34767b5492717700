"""MI355X-native DEER / quasi-DEER Newton evaluation of nonlinear RNNs.

The compute path is the HIP library ``libpararnn.so`` behind the C ABI in
``include/pararnn.h``; ``nonlinear_rnn_evaluation_newton_amd.binding`` is the
thin Python front end (argument marshalling only).  Importing this package
does not load the library; ``binding.lib()`` does, and raises if it is
missing.
"""
__all__ = ["binding", "synthetic"]
