// qmv_k_mxfp4i.hip -- kernel instantiations for MXFP4 weights with int8
// activations (one translation unit per format so the build runs in
// parallel; built once per workgroup size, see QMV_NS in qmv_device.hpp).
#include "qmv_device.hpp"

namespace QMV_NS {
extern const void *const kTable_mxfp4i[3][4][5];
const void *const kTable_mxfp4i[3][4][5] = QMV_TABLE(kMXFP4I, false);
extern const void *const kTableGU_mxfp4i[2][4][5];
const void *const kTableGU_mxfp4i[2][4][5] = QMV_TABLE_GU(kMXFP4I, false);
extern const void *const kTableCB_mxfp4i[4][4];
const void *const kTableCB_mxfp4i[4][4] = QMV_TABLE_CB(kMXFP4I, false);
#if QMV_WAVES == 4     // grouped kernels: 4-wave workgroups
extern const void *const kTableGR_mxfp4i[2][4][5];
const void *const kTableGR_mxfp4i[2][4][5] = QMV_TABLE_GR(kMXFP4I, false);
#endif
}  // namespace QMV_NS
