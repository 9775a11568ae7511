// The persistent kernel, the kernel-per-operator baseline and the body timer
// for batch 2..16: the same runtime and task bodies as megakernel.hip,
// compiled with MPK_BN = 1 as kernels of their own (mpk_megakernel_bn,
// mpk_baseline_op_bn, mpk_time_task_kernel_bn), so that the batch > 1 paths
// can change without changing the batch-1 kernel's code.
#define MPK_BN 1
#include "megakernel.hip"
