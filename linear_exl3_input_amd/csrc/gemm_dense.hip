// Dense GEMM over dequantized B fragments (all widths and codebooks).
#include "exl3_gemm_dense.hpp"
