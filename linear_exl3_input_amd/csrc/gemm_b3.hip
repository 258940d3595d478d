// Trellis GEMM and decode kernels for 3-bit weights (all codebooks).
#include "exl3_gemm_wide.hpp"
#include "exl3_gemm_lut.hpp"
EXL3_DEFINE_BITS(3)
