// qmv_k_mxfp4.hip -- kernel instantiations for one weight format (split into
// one translation unit per format so the build runs in parallel).
#include "qmv_device.hpp"

namespace qmv {
extern const void *const kTable_mxfp4[3][4][5];
const void *const kTable_mxfp4[3][4][5] = QMV_TABLE(kMXFP4);
extern const void *const kTableGU_mxfp4[2][4][5];
const void *const kTableGU_mxfp4[2][4][5] = QMV_TABLE_GU(kMXFP4);
}  // namespace qmv
