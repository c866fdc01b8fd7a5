"""MI355X-native FlashAttention-2 forward: a C-ABI HIP library plus a thin binding.

The binding (``exact_attention_22_amd.fa``) loads ``libfa.so`` on first use and
raises if it is missing; nothing here falls back to a CPU or PyTorch path.
"""
