// W4A8 prefill grouped GEMM (block-scaled FP4 x FP8 matrix instructions).
#include "moeq_device.h"
#include "moeq_kernels.h"
