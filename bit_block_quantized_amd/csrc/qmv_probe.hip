// qmv_probe.hip -- read-only streaming probe (include/qmv_probe.h).
//
// Each workgroup reads one chunk of THREADS * PER * 16 bytes of one region
// with 16-byte raw buffer loads carrying the non-temporal hint, the same
// load form the GEMV kernels use for codes.  Chunks are numbered over all
// regions in order; a workgroup finds its region from the chunk prefix sums
// (kernel arguments, read with scalar loads).
#include "qmv_probe.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct ProbeArgs {
    const uint8_t *p[QMV_PROBE_MAX_REGIONS];
    uint32_t bytes[QMV_PROBE_MAX_REGIONS];
    uint32_t first_chunk[QMV_PROBE_MAX_REGIONS + 1];   // prefix sums of chunks per region
    int n;
    unsigned *sink;
};

constexpr uint32_t kSinkKey = 0x9E3779B9u;

template <int THREADS, int PER>
__global__ __launch_bounds__(THREADS) void stream_read(const ProbeArgs a)
{
    const uint32_t chunk = blockIdx.x;
    int r = 0;
    while (r + 1 < a.n && chunk >= a.first_chunk[r + 1]) ++r;      // uniform per workgroup
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(a.p[r]), (short)0, (int)a.bytes[r], 0x00020000);
    const uint32_t off = (chunk - a.first_chunk[r]) * (uint32_t)(THREADS * PER * 16) + threadIdx.x * 16u;
    u32x4 v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i)
        v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, off + i * THREADS * 16, 0, 2);
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
    if (acc == kSinkKey) a.sink[0] = acc;
}

struct Shape { const void *fn; int threads, per; };

const Shape kShapes[QMV_PROBE_VARIANTS] = {
    {(const void *)&stream_read<256, 4>, 256, 4},
    {(const void *)&stream_read<256, 8>, 256, 8},
    {(const void *)&stream_read<512, 4>, 512, 4},
    {(const void *)&stream_read<512, 8>, 512, 8},
    {(const void *)&stream_read<1024, 2>, 1024, 2},
    {(const void *)&stream_read<1024, 4>, 1024, 4},
};

// One thread stores the GPU's constant-rate real-time counter (100 MHz on
// this device) with a vector store.
__global__ __launch_bounds__(64) void clock_stamp(unsigned long long *out)
{
    if (threadIdx.x == 0) *out = __builtin_amdgcn_s_memrealtime();
}

}  // namespace

extern "C" {

__attribute__((visibility("default")))
qmv_status_t qmv_probe_clock(unsigned long long *out, hipStream_t stream)
{
    if (!out || ((uintptr_t)out & 7))
        return QMV_EINVAL;
    void *kargs[] = {&out};
    if (hipLaunchKernel((const void *)&clock_stamp, dim3(1), dim3(64), kargs, 0, stream) != hipSuccess)
        return QMV_EHIP;
    return QMV_OK;
}

__attribute__((visibility("default")))
qmv_status_t qmv_probe_stream_read(int n_regions, const void *const *ptrs,
                                   const long long *bytes, int variant, unsigned *sink,
                                   hipStream_t stream)
{
    if (!ptrs || !bytes || !sink || ((uintptr_t)sink & 3))
        return QMV_EINVAL;
    if (n_regions < 1 || n_regions > QMV_PROBE_MAX_REGIONS || variant < 0 ||
        variant >= QMV_PROBE_VARIANTS)
        return QMV_EUNSUPPORTED;
    const Shape &sh = kShapes[variant];
    const long long chunk_bytes = (long long)sh.threads * sh.per * 16;
    ProbeArgs a;
    a.n = n_regions;
    a.sink = sink;
    long long chunks = 0;
    for (int r = 0; r < n_regions; ++r) {
        if (!ptrs[r] || ((uintptr_t)ptrs[r] & 15) || bytes[r] < 1 || bytes[r] >= (1LL << 31))
            return QMV_EINVAL;
        a.p[r] = (const uint8_t *)ptrs[r];
        a.bytes[r] = (uint32_t)bytes[r];
        a.first_chunk[r] = (uint32_t)chunks;
        chunks += (bytes[r] + chunk_bytes - 1) / chunk_bytes;
    }
    a.first_chunk[n_regions] = (uint32_t)chunks;
    for (int r = n_regions; r < QMV_PROBE_MAX_REGIONS; ++r) {
        a.p[r] = nullptr;
        a.bytes[r] = 0;
        a.first_chunk[r + 1] = (uint32_t)chunks;
    }
    if (chunks >= (1LL << 31))
        return QMV_EINVAL;
    void *kargs[] = {&a};
    if (hipLaunchKernel(sh.fn, dim3((unsigned)chunks), dim3(sh.threads), kargs, 0, stream) !=
        hipSuccess)
        return QMV_EHIP;
    return QMV_OK;
}

}  // extern "C"
