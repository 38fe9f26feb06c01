// MFMA grouped GEMM (to come).
#include "common.h"
