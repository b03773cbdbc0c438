// Grouped (prefill) path: MFMA kernels, added next.
#include "common.hpp"
#include "internal.hpp"
