// qmv_k_cb2s.hip -- kernel instantiations for one weight format (split into
// one translation unit per format so the build runs in parallel; built once
// per workgroup size, see QMV_NS in qmv_device.hpp).
#include "qmv_device.hpp"

namespace QMV_NS {
extern const void *const kTable_cb2s[3][4][5];
const void *const kTable_cb2s[3][4][5] = QMV_TABLE(kCB2S, false);
extern const void *const kTableGU_cb2s[2][4][5];
const void *const kTableGU_cb2s[2][4][5] = QMV_TABLE_GU(kCB2S, false);
extern const void *const kTableCB_cb2s[4][4];
const void *const kTableCB_cb2s[4][4] = QMV_TABLE_CB(kCB2S, false);
#if QMV_WAVES == 4     // grouped kernels: 4-wave workgroups
extern const void *const kTableGR_cb2s[2][4][5];
const void *const kTableGR_cb2s[2][4][5] = QMV_TABLE_GR(kCB2S, false);
#endif
}  // namespace QMV_NS
