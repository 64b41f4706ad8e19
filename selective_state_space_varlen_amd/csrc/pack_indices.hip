// varlen_pack_indices: cu_seqlens -> position_indices and head flags.
//
// Shanghai AI Lab article on packed variable-length Mamba-1 training
// (gitcode.csdn.net/69d8cc1b54b52172bc6872cb.html), section "conv1d_pack 算子",
// figure (a): pack() emits each token's position inside its own sequence.
// One thread per token finds its sequence by binary search over cu_seqlens
// (a few hundred bytes, L1/L2 resident); a single extra workgroup validates
// cu_seqlens and writes its status word, so no memory needs clearing beforehand.
#include "common.h"

namespace ssmp {

__global__ __launch_bounds__(256) void k_pack_indices(const int32_t* __restrict__ cu, int32_t nseq, int64_t T,
                                                      int32_t* __restrict__ pos, uint8_t* __restrict__ heads) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < T; t += stride) {
        // largest s in [0, nseq-1] with cu[s] <= t
        int lo = 0, hi = nseq - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if ((int64_t)cu[mid] <= t) lo = mid; else hi = mid - 1;
        }
        int64_t p = t - (int64_t)cu[lo];
        // keep 0 <= pos <= t even for an invalid cu_seqlens, so that no
        // consumer can be steered out of bounds
        if (p < 0) p = 0;
        if (p > t) p = t;
        pos[t] = (int32_t)p;
        if (heads) heads[t] = (p == 0) ? 1 : 0;
    }
}

__global__ __launch_bounds__(256) void k_validate_cu(const int32_t* __restrict__ cu, int32_t nseq, int64_t T,
                                                     int32_t* __restrict__ err) {
    int bad = 0;
    for (int i = threadIdx.x; i < nseq; i += blockDim.x)
        if (cu[i + 1] < cu[i]) bad = 1;
    if (threadIdx.x == 0 && (cu[0] != 0 || (int64_t)cu[nseq] != T)) bad = 1;
    bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) *err = bad ? SSMP_ERR_CU_SEQLENS : SSMP_OK;
}

}  // namespace ssmp

extern "C" int varlen_pack_indices(const int32_t* cu_seqlens, int32_t nseq, int64_t T, int32_t* pos,
                                   uint8_t* heads, int32_t* dev_err, void* stream) {
    using namespace ssmp;
    if (nseq < 1 || T < 0 || T >= (int64_t(1) << 31)) return SSMP_ERR_SHAPE;
    if (!cu_seqlens) return SSMP_ERR_NULL;
    if (T > 0 && !pos) return SSMP_ERR_NULL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dev_err) {
        k_validate_cu<<<1, 256, 0, s>>>(cu_seqlens, nseq, T, dev_err);
        SSMP_LAUNCH_CHECK();
    }
    if (T > 0) {
        int64_t blocks = (T + 255) / 256;
        if (blocks > 8192) blocks = 8192;
        k_pack_indices<<<(unsigned)blocks, 256, 0, s>>>(cu_seqlens, nseq, T, pos, heads);
        SSMP_LAUNCH_CHECK();
    }
    return SSMP_OK;
}

extern "C" const char* ssmp_status_string(int status) {
    switch (status) {
        case SSMP_OK: return "ok";
        case SSMP_ERR_NULL: return "a required pointer is NULL";
        case SSMP_ERR_SHAPE: return "a size is out of range or sizes overflow";
        case SSMP_ERR_CU_SEQLENS: return "cu_seqlens is invalid (cu[0] != 0, decreasing, or cu[nseq] != T)";
        case SSMP_ERR_UNSUPPORTED: return "dtype, d_state or conv width not supported";
        case SSMP_ERR_HIP: return "a HIP kernel launch failed";
        case SSMP_ERR_WORKSPACE: return "workspace missing or too small";
        case SSMP_ERR_TOO_LARGE: return "the problem needs more scratch than the library's own buffer holds";
        default: return "unknown status";
    }
}

extern "C" int ssmp_abi_version(void) { return 6; }
