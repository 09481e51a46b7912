"""MI355X-native multi-LoRA add-on (SGMV / BGMV shrink and expand) on hand-written HIP kernels.

The compute path is the C-ABI library ``liblora_sgmv.so`` (see ``include/lora_sgmv.h``);
``segmented_gather_matmul_amd.binding`` marshals torch tensors into it.  Importing this
package loads nothing: the binding loads the library on first use and raises if it is
missing.
"""
