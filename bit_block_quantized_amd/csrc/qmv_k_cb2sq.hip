// qmv_k_cb2sq.hip -- kernel instantiations for one weight format fed bf16
// activations that are quantized to int8 blocks while staged (one
// translation unit per format so the build runs in parallel; built once per
// workgroup size, see QMV_NS in qmv_device.hpp).
#include "qmv_device.hpp"

namespace QMV_NS {
extern const void *const kTableQ_cb2s[3][4][5];
const void *const kTableQ_cb2s[3][4][5] = QMV_TABLE(kCB2S, true);
extern const void *const kTableQGU_cb2s[2][4][5];
const void *const kTableQGU_cb2s[2][4][5] = QMV_TABLE_GU(kCB2S, true);
extern const void *const kTableQCB_cb2s[4][4];
const void *const kTableQCB_cb2s[4][4] = QMV_TABLE_CB(kCB2S, true);
#if QMV_WAVES == 4     // grouped kernels: 4-wave workgroups
extern const void *const kTableQGR_cb2s[2][4][5];
const void *const kTableQGR_cb2s[2][4][5] = QMV_TABLE_GR(kCB2S, true);
#endif
}  // namespace QMV_NS
