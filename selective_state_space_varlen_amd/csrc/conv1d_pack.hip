// conv1d_pack forward and backward: causal depthwise conv of width W <= 4 that
// stops at each sequence's head token.
//
// Shanghai AI Lab article on packed variable-length Mamba-1 training
// (gitcode.csdn.net/69d8cc1b54b52172bc6872cb.html), section "conv1d_pack 算子":
// the conv looks back W-1 tokens and terminates early at a head; the backward
// stops dx and dweight the same way, taking the reverse position from the
// position index W-1 tokens ahead.
//
// Both kernels stream HBM: a thread owns V adjacent channels (one 16-byte
// vector) and a run of RT consecutive tokens, slides a W-token window of x in
// registers, and reads the per-token position once per token (the same
// address for the whole wave). Consecutive lanes own consecutive vectors, so
// a wave reads 1 KiB of one row per load.
#include "common.h"

namespace ssmp {

template <typename T>
struct Vec;
template <>
struct Vec<uint16_t> {
    static constexpr int V = 8;
    using raw = uint4;
    static __device__ __forceinline__ void unpack(const raw& r, float (&f)[V]) {
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = bf16_to_f32(w[i]);
            f[2 * i + 1] = bf16_hi_to_f32(w[i]);
        }
    }
    static __device__ __forceinline__ raw pack(const float (&f)[V]) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = (uint32_t)f32_to_bf16(f[2 * i]) | ((uint32_t)f32_to_bf16(f[2 * i + 1]) << 16);
        return make_uint4(w[0], w[1], w[2], w[3]);
    }
};
template <>
struct Vec<float> {
    static constexpr int V = 4;
    using raw = float4;
    static __device__ __forceinline__ void unpack(const raw& r, float (&f)[V]) {
        f[0] = r.x; f[1] = r.y; f[2] = r.z; f[3] = r.w;
    }
    static __device__ __forceinline__ raw pack(const float (&f)[V]) { return make_float4(f[0], f[1], f[2], f[3]); }
};

// Scalar fallback when D is not a multiple of the vector width.
template <typename T>
struct Vec1 {
    static constexpr int V = 1;
};

template <typename T, bool VEC>
struct Access {
    static constexpr int V = VEC ? Vec<T>::V : 1;
    static __device__ __forceinline__ void load(const T* __restrict__ p, float (&f)[V]) {
        if constexpr (VEC) {
            Vec<T>::unpack(*reinterpret_cast<const typename Vec<T>::raw*>(p), f);
        } else {
            f[0] = Elt<T>::ld(p, 0);
        }
    }
    static __device__ __forceinline__ void store(T* __restrict__ p, const float (&f)[V]) {
        if constexpr (VEC) {
            *reinterpret_cast<typename Vec<T>::raw*>(p) = Vec<T>::pack(f);
        } else {
            Elt<T>::st(p, 0, f[0]);
        }
    }
};

constexpr int kConvFwdRun = 32;   // tokens per thread, forward
constexpr int kConvBwdRun = 128;  // tokens per thread, backward (sets the partial-sum count)

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
template <typename T, bool VEC>
__global__ __launch_bounds__(256) void k_conv_fwd(const T* __restrict__ x, const float* __restrict__ w,
                                                  const float* __restrict__ b, const int32_t* __restrict__ pos,
                                                  T* __restrict__ u, int64_t T_, int D, int W, int silu) {
    using A = Access<T, VEC>;
    constexpr int V = A::V;
    const int nvec = D / V;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int cv = (int)(gid % nvec);
    const int64_t t0 = (gid / nvec) * kConvFwdRun;
    if (t0 >= T_) return;
    const int64_t t1 = (t0 + kConvFwdRun < T_) ? t0 + kConvFwdRun : T_;
    const int d0 = cv * V;

    // wk[k][i]: weight of the tap k tokens back, for channel d0+i (0 beyond W)
    float wk[4][V], bias[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        bias[i] = b ? b[d0 + i] : 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k) wk[k][i] = (k < W) ? w[(size_t)(d0 + i) * W + (W - 1 - k)] : 0.0f;
    }
    // window xw[k] = x[t-k]; tokens before 0 are never selected
    float xw[4][V];
#pragma unroll
    for (int k = 1; k < 4; ++k) {
        const int64_t tk = t0 - k;
        if (tk >= 0) {
            A::load(x + (size_t)tk * D + d0, xw[k]);
        } else {
#pragma unroll
            for (int i = 0; i < V; ++i) xw[k][i] = 0.0f;
        }
    }
    for (int64_t t = t0; t < t1; ++t) {
        A::load(x + (size_t)t * D + d0, xw[0]);
        int kmax = pos[t];
        if (kmax > W - 1) kmax = W - 1;
        if ((int64_t)kmax > t) kmax = (int)t;
        float o[V];
#pragma unroll
        for (int i = 0; i < V; ++i) {
            float acc = bias[i];
#pragma unroll
            for (int k = 0; k < 4; ++k) acc += (k <= kmax) ? wk[k][i] * xw[k][i] : 0.0f;
            o[i] = silu ? acc * sigmoid_fast(acc) : acc;
        }
        A::store(u + (size_t)t * D + d0, o);
#pragma unroll
        for (int k = 3; k > 0; --k)
#pragma unroll
            for (int i = 0; i < V; ++i) xw[k][i] = xw[k - 1][i];
    }
}

// ---------------------------------------------------------------------------
// backward
// ---------------------------------------------------------------------------
// Per thread: tokens [t0, t1). gv[t] = du[t] * act'(v[t]) is produced for
// t in [t0, min(t1 + 3, T)); dx[s] for s in [t0, t1) collects
// sum_k [k <= pos[s+k]] w[W-1-k] gv[s+k]; dw and db partial sums over
// [t0, t1) go to part[run][j][d] (j = tap k for k < 4, j = 4 for the bias).
template <typename T, bool VEC>
__global__ __launch_bounds__(256) void k_conv_bwd(const T* __restrict__ x, const float* __restrict__ w,
                                                  const float* __restrict__ b, const int32_t* __restrict__ pos,
                                                  const T* __restrict__ du, T* __restrict__ dx,
                                                  float* __restrict__ part, int64_t T_, int D, int W, int silu) {
    using A = Access<T, VEC>;
    constexpr int V = A::V;
    const int nvec = D / V;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int cv = (int)(gid % nvec);
    const int64_t run = gid / nvec;
    const int64_t t0 = run * kConvBwdRun;
    if (t0 >= T_) return;
    const int64_t t1 = (t0 + kConvBwdRun < T_) ? t0 + kConvBwdRun : T_;
    const int64_t tend = (t1 + 3 < T_) ? t1 + 3 : T_;
    const int d0 = cv * V;

    float wk[4][V], bias[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        bias[i] = b ? b[d0 + i] : 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k) wk[k][i] = (k < W) ? w[(size_t)(d0 + i) * W + (W - 1 - k)] : 0.0f;
    }
    float xw[4][V];
#pragma unroll
    for (int k = 1; k < 4; ++k) {
        const int64_t tk = t0 - k;
        if (tk >= 0) {
            A::load(x + (size_t)tk * D + d0, xw[k]);
        } else {
#pragma unroll
            for (int i = 0; i < V; ++i) xw[k][i] = 0.0f;
        }
    }
    // gq[j][i] = gv[t-j] masked for the dx contribution of tap j:
    // gq[j] = [j <= kmax(t-j)] * gv[t-j]; kept for j = 0..3
    float gq[4][4][V];  // [age j][tap k][i]: contribution of token t-j to dx[t-j-k]
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int i = 0; i < V; ++i) gq[j][k][i] = 0.0f;
    float dwp[4][V], dbp[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        dbp[i] = 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k) dwp[k][i] = 0.0f;
    }

    for (int64_t t = t0; t < tend + 3; ++t) {
        // shift ages
#pragma unroll
        for (int j = 3; j > 0; --j)
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int i = 0; i < V; ++i) gq[j][k][i] = gq[j - 1][k][i];
        if (t < tend) {
            A::load(x + (size_t)t * D + d0, xw[0]);
            float g[V];
            A::load(du + (size_t)t * D + d0, g);
            int kmax = pos[t];
            if (kmax > W - 1) kmax = W - 1;
            if ((int64_t)kmax > t) kmax = (int)t;
            const bool own = t < t1;  // dw/db sums only over this thread's tokens
#pragma unroll
            for (int i = 0; i < V; ++i) {
                float v = bias[i];
#pragma unroll
                for (int k = 0; k < 4; ++k) v += (k <= kmax) ? wk[k][i] * xw[k][i] : 0.0f;
                float gv = g[i];
                if (silu) {
                    const float s = sigmoid_fast(v);
                    gv = g[i] * s * (1.0f + v * (1.0f - s));
                }
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const bool on = k <= kmax;
                    gq[0][k][i] = on ? gv : 0.0f;
                    if (own && on) dwp[k][i] += gv * xw[k][i];
                }
                if (own) dbp[i] += gv;
            }
#pragma unroll
            for (int k = 3; k > 0; --k)
#pragma unroll
                for (int i = 0; i < V; ++i) xw[k][i] = xw[k - 1][i];
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int i = 0; i < V; ++i) gq[0][k][i] = 0.0f;
        }
        // dx[t-3] = sum_k w_k * gq[age 3-k][tap k]  (token t-3+k feeds tap k)
        const int64_t s = t - 3;
        if (s >= t0 && s < t1) {
            float o[V];
#pragma unroll
            for (int i = 0; i < V; ++i) {
                float acc = 0.0f;
#pragma unroll
                for (int k = 0; k < 4; ++k) acc += wk[k][i] * gq[3 - k][k][i];
                o[i] = acc;
            }
            A::store(dx + (size_t)s * D + d0, o);
        }
    }
#pragma unroll
    for (int i = 0; i < V; ++i) {
#pragma unroll
        for (int k = 0; k < 4; ++k) part[((size_t)run * 5 + k) * D + d0 + i] = dwp[k][i];
        part[((size_t)run * 5 + 4) * D + d0 + i] = dbp[i];
    }
}

// dw[d, W-1-k] = sum_run part[run][k][d];  db[d] = sum_run part[run][4][d]
__global__ __launch_bounds__(256) void k_conv_bwd_reduce(const float* __restrict__ part, int64_t nrun, int D, int W,
                                                         float* __restrict__ dw, float* __restrict__ db) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)5 * D) return;
    const int j = (int)(i / D), d = (int)(i % D);
    if (j < 4 && j >= W) return;
    if (j == 4 && !db) return;
    float acc = 0.0f;
    for (int64_t r = 0; r < nrun; ++r) acc += part[((size_t)r * 5 + j) * D + d];
    if (j < 4) dw[(size_t)d * W + (W - 1 - j)] = acc;
    else db[d] = acc;
}

static bool vec_ok(const void* p, int D, int V) {
    return (D % V == 0) && ((reinterpret_cast<uintptr_t>(p) & 15u) == 0);
}

template <typename T>
static int launch_fwd(const void* x, const float* w, const float* b, const int32_t* pos, void* u, int64_t T_, int D,
                      int W, int silu, hipStream_t s) {
    const bool vec = vec_ok(x, D, Vec<T>::V) && vec_ok(u, D, Vec<T>::V);
    const int V = vec ? Vec<T>::V : 1;
    const int64_t nthreads = (int64_t)(D / V) * ((T_ + kConvFwdRun - 1) / kConvFwdRun);
    const int64_t blocks = (nthreads + 255) / 256;
    if (blocks > 0x7fffffff) return SSMP_ERR_SHAPE;
    if (vec)
        k_conv_fwd<T, true><<<(unsigned)blocks, 256, 0, s>>>((const T*)x, w, b, pos, (T*)u, T_, D, W, silu);
    else
        k_conv_fwd<T, false><<<(unsigned)blocks, 256, 0, s>>>((const T*)x, w, b, pos, (T*)u, T_, D, W, silu);
    SSMP_LAUNCH_CHECK();
    return SSMP_OK;
}

template <typename T>
static int launch_bwd(const void* x, const float* w, const float* b, const int32_t* pos, const void* du, void* dx,
                      float* dw, float* db, float* part, int64_t T_, int D, int W, int silu, hipStream_t s) {
    const bool vec = vec_ok(x, D, Vec<T>::V) && vec_ok(du, D, Vec<T>::V) && vec_ok(dx, D, Vec<T>::V);
    const int V = vec ? Vec<T>::V : 1;
    const int64_t nrun = (T_ + kConvBwdRun - 1) / kConvBwdRun;
    const int64_t nthreads = (int64_t)(D / V) * nrun;
    const int64_t blocks = (nthreads + 255) / 256;
    if (blocks > 0x7fffffff) return SSMP_ERR_SHAPE;
    if (vec)
        k_conv_bwd<T, true><<<(unsigned)blocks, 256, 0, s>>>((const T*)x, w, b, pos, (const T*)du, (T*)dx, part, T_,
                                                               D, W, silu);
    else
        k_conv_bwd<T, false><<<(unsigned)blocks, 256, 0, s>>>((const T*)x, w, b, pos, (const T*)du, (T*)dx, part, T_,
                                                                D, W, silu);
    SSMP_LAUNCH_CHECK();
    k_conv_bwd_reduce<<<(unsigned)((5 * (int64_t)D + 255) / 256), 256, 0, s>>>(part, nrun, D, W, dw, db);
    SSMP_LAUNCH_CHECK();
    return SSMP_OK;
}

static int check_conv_args(int64_t T_, int D, int W, int dtype) {
    if (T_ < 0 || D < 1) return SSMP_ERR_SHAPE;
    if (T_ > 0 && (T_ * (int64_t)D) >= (int64_t(1) << 40)) return SSMP_ERR_SHAPE;
    if (W < 1 || W > 4) return SSMP_ERR_UNSUPPORTED;
    if (dtype != SSMP_F32 && dtype != SSMP_BF16) return SSMP_ERR_UNSUPPORTED;
    return SSMP_OK;
}

}  // namespace ssmp

extern "C" int conv1d_pack_fwd(const void* x, const float* w, const float* b, const int32_t* pos, void* u,
                               int64_t T, int32_t D, int32_t W, int32_t dtype, int32_t silu, void* stream) {
    using namespace ssmp;
    int st = check_conv_args(T, D, W, dtype);
    if (st) return st;
    if (T == 0) return SSMP_OK;
    if (!x || !w || !pos || !u) return SSMP_ERR_NULL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return dtype == SSMP_BF16 ? launch_fwd<uint16_t>(x, w, b, pos, u, T, D, W, silu != 0, s)
                              : launch_fwd<float>(x, w, b, pos, u, T, D, W, silu != 0, s);
}

extern "C" size_t conv1d_pack_bwd_workspace_bytes(int64_t T, int32_t D, int32_t W) {
    (void)W;
    if (T <= 0 || D <= 0) return 0;
    const int64_t nrun = (T + ssmp::kConvBwdRun - 1) / ssmp::kConvBwdRun;
    return (size_t)nrun * 5 * (size_t)D * sizeof(float);
}

extern "C" int conv1d_pack_bwd(const void* x, const float* w, const float* b, const int32_t* pos, const void* du,
                               void* dx, float* dw, float* db, void* workspace, size_t workspace_bytes, int64_t T,
                               int32_t D, int32_t W, int32_t dtype, int32_t silu, void* stream) {
    using namespace ssmp;
    int st = check_conv_args(T, D, W, dtype);
    if (st) return st;
    if (!w || !dw) return SSMP_ERR_NULL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (T == 0) {
        // empty input: the sums are zero
        if (hipMemsetAsync(dw, 0, sizeof(float) * (size_t)D * W, s) != hipSuccess) return SSMP_ERR_HIP;
        if (db && hipMemsetAsync(db, 0, sizeof(float) * (size_t)D, s) != hipSuccess) return SSMP_ERR_HIP;
        return SSMP_OK;
    }
    if (!x || !pos || !du || !dx) return SSMP_ERR_NULL;
    if (!workspace || workspace_bytes < conv1d_pack_bwd_workspace_bytes(T, D, W)) return SSMP_ERR_WORKSPACE;
    return dtype == SSMP_BF16
               ? launch_bwd<uint16_t>(x, w, b, pos, du, dx, dw, db, (float*)workspace, T, D, W, silu != 0, s)
               : launch_bwd<float>(x, w, b, pos, du, dx, dw, db, (float*)workspace, T, D, W, silu != 0, s);
}
