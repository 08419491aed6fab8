// row_inst.hip -- instantiations of the row-per-lane forward kernel
// (scan_row.h) for one element type and one input-term rule, selected by
// compile definitions (build.py compiles this file four times):
//   MSCAN_INST_BF16  = 1 (bfloat16 tensors) or 0 (float32)
//   MSCAN_INST_EXACT = 1 (exact zero-order hold) or 0 (Δ·B·u)
#define MSCAN_INSTANTIATE_ROWS
#include "scan_launch.h"

#if !defined(MSCAN_INST_BF16) || !defined(MSCAN_INST_EXACT)
#error "MSCAN_INST_BF16 and MSCAN_INST_EXACT must be defined"
#endif

#if MSCAN_INST_BF16
#define MSCAN_TIN uint16_t
#define MSCAN_T_NAME bf16
#else
#define MSCAN_TIN float
#define MSCAN_T_NAME f32
#endif
#if MSCAN_INST_EXACT
#define MSCAN_R_NAME exact
#else
#define MSCAN_R_NAME simple
#endif
#define MSCAN_CAT3(a, b, c) a##_##b##_##c
#define MSCAN_NAME(a, b, c) MSCAN_CAT3(a, b, c)

namespace mscan {

int MSCAN_NAME(dispatch_rows, MSCAN_T_NAME, MSCAN_R_NAME)(const ScanParams& p, const Plan& pl, hipStream_t s) {
  return dispatch_rows<MSCAN_TIN, MSCAN_INST_EXACT != 0>(p, pl, s);
}

}  // namespace mscan
